"""The C ABI driven from plain C: tests/c_driver.c (C99, the HIP runtime's C API for memory
and streams, libh2o.so for every H2O call) runs a reset, a prefill and decode steps; every
result must equal, bit for bit, the same calls made through the Python binding, whose
results the other GPU tests check against the oracle."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest
import torch

from workloads import Workload, generate

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu


def _compile(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    from kv_cache_eviction_03_amd._abi import LIB_PATH
    lib_dir = os.path.dirname(LIB_PATH)
    exe = tmp_path / "c_driver"
    # the HIP runtime header as a system header: -pedantic applies to this program only
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-isystem", "/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "c_driver.c"), "-o", str(exe),
           f"-L{lib_dir}", "-lh2o", f"-Wl,-rpath,{lib_dir}",
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("dtype,code", [("f16", 1), ("bf16", 2)])
def test_c_program_matches_the_binding(tmp_path, dtype, code):
    from kv_cache_eviction_03_amd import H2OCache
    exe = _compile(tmp_path)
    w = Workload(62, f"c-driver-{dtype}", 2, 1, 3, 128, dtype, 200, 12, 24, 16, heavy_frac=0.05)
    B, H, d, T, n = w.batch, w.heads, w.head_dim, w.prompt, w.steps
    print(f"[c-driver] {w.name}: B {B}, H {H}, d {d}, T {T}, {n} steps", flush=True)
    x = generate(w, seed=3)
    for name in ("q_prompt", "k_prompt", "v_prompt", "q_dec", "k_dec", "v_dec"):
        (tmp_path / f"{name}.bin").write_bytes(x[name].contiguous().view(torch.int16).numpy().tobytes())
    r = subprocess.run([str(exe), str(tmp_path), str(B), str(H), str(d), str(w.k_heavy),
                        str(w.k_local), str(code), str(T), str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    # the same calls through the binding
    g = {k: v.to("cuda") for k, v in x.items()}
    c = H2OCache(B, H, d, w.k_heavy, w.k_local, w.torch_dtype, "cuda", max_prompt=T)
    c.reset()
    out_p, cs = c.prefill(g["q_prompt"], g["k_prompt"], g["v_prompt"])
    outs = torch.empty((n, B, H, d), dtype=torch.float32, device="cuda")
    vic = torch.empty((n, B, H), dtype=torch.int32, device="cuda")
    evp = torch.empty((n, B, H), dtype=torch.int32, device="cuda")
    eva = torch.empty((n, B, H), dtype=torch.float32, device="cuda")
    for i in range(n):
        c.decode(g["q_dec"][i], g["k_dec"][i], g["v_dec"][i], out=outs[i], victim_slot=vic[i],
                 evicted_pos=evp[i], evicted_acc=eva[i])
    torch.cuda.synchronize()

    def raw(t):
        return t.contiguous().cpu().view(torch.uint8).numpy().tobytes()

    expect = {"prefill_out.bin": out_p, "colsum.bin": cs, "dec_out.bin": outs,
              "victims.bin": vic, "ev_pos.bin": evp, "ev_acc.bin": eva,
              "slot_pos.bin": c.slot_pos, "acc.bin": c.acc_score,
              "k_slots.bin": c.k_slots, "v_slots.bin": c.v_slots}
    for name, t in expect.items():
        got = (tmp_path / name).read_bytes()
        assert got == raw(t), name
    # the run evicted: every unit's cache was full during the decode steps
    assert (vic >= 0).all()
