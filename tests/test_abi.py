"""The C ABI without a GPU: symbols, workspace sizing and argument checks.

Every rejected call must return its status before any HIP call, so these run
on a machine with no device. Pointers here are fake, aligned integers: a call
that passed validation would try to launch, which none of these do.
"""
import os
import re

import pytest

import kv_cache_eviction_03_amd as h2o
from kv_cache_eviction_03_amd import CacheDesc, DecodeAux

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000          # a 256-byte aligned fake device address


def header_functions():
    text = open(os.path.join(ROOT, "include", "h2o.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(h2o_\w+)\s*\(", text, re.M)))


def desc(**kw):
    d = dict(batch=2, heads=3, head_dim=128, k_heavy=4, k_local=4, dtype=h2o.H2O_F16,
             k_slots=A, v_slots=A + 0x1000, slot_pos=A + 0x2000, acc_score=A + 0x3000)
    d.update(kw)
    return CacheDesc(**d)


def test_library_exports_every_declared_function():
    lib = h2o.library()
    declared = header_functions()
    assert declared == sorted(h2o.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    assert h2o.h2o_status_str(h2o.H2O_OK) == "H2O_OK"
    assert h2o.h2o_status_str(h2o.H2O_ERR_WORKSPACE) == "H2O_ERR_WORKSPACE"


def round256(n):
    return (n + 255) // 256 * 256


def test_workspace_bytes():
    d = desc()
    units, T = 2 * 3, 512
    # fp16/bf16: partial column-sum rows of 128, 256, 384 and 512 keys (one per
    # 128-row query block), then the column sums
    assert h2o.h2o_workspace_bytes(d, T) == (round256(units * (128 + 256 + 384 + 512) * 4)
                                             + round256(units * T * 4))
    # ragged last block: 128 + 256 + 300 keys
    assert h2o.h2o_workspace_bytes(d, 300) == (round256(units * (128 + 256 + 300) * 4)
                                               + round256(units * 300 * 4))
    # fp32: row log-sum-exps, one partial row of T keys, the column sums
    assert h2o.h2o_workspace_bytes(desc(dtype=h2o.H2O_F32), T) == 3 * round256(units * T * 4)
    sizes = [h2o.h2o_workspace_bytes(d, t) for t in range(0, 1200, 37)]
    assert sizes == sorted(sizes)                 # a workspace for T serves every shorter prompt
    assert h2o.h2o_workspace_bytes(d, 0) == 0
    assert h2o.h2o_workspace_bytes(d, -1) == 0
    assert h2o.h2o_workspace_bytes(desc(head_dim=96), 16) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), h2o.H2O_ERR_INVALID),
    (dict(heads=-1), h2o.H2O_ERR_INVALID),
    (dict(dtype=7), h2o.H2O_ERR_INVALID),
    (dict(head_dim=96), h2o.H2O_ERR_UNSUPPORTED),
    (dict(k_local=0), h2o.H2O_ERR_INVALID),
    (dict(k_heavy=-1), h2o.H2O_ERR_INVALID),
    (dict(k_heavy=h2o.H2O_MAX_SLOTS), h2o.H2O_ERR_UNSUPPORTED),
    (dict(k_slots=0), h2o.H2O_ERR_INVALID),
    (dict(acc_score=0), h2o.H2O_ERR_INVALID),
    (dict(v_slots=A + 8), h2o.H2O_ERR_INVALID),
    (dict(slot_pos=A + 2), h2o.H2O_ERR_INVALID),
    (dict(policy=4), h2o.H2O_ERR_INVALID),
    (dict(policy=-1), h2o.H2O_ERR_INVALID),
    (dict(policy=2, policy_param=0), h2o.H2O_ERR_INVALID),
    (dict(policy=1, policy_param=-1), h2o.H2O_ERR_INVALID),
    (dict(slot_format=2), h2o.H2O_ERR_INVALID),
    (dict(slot_format=-1), h2o.H2O_ERR_INVALID),
    (dict(slot_format=1, dtype=h2o.H2O_F32, k_scale=1.0, v_scale=1.0), h2o.H2O_ERR_UNSUPPORTED),
    (dict(slot_format=1, k_scale=0.0, v_scale=1.0), h2o.H2O_ERR_INVALID),
    (dict(slot_format=1, k_scale=1.0, v_scale=-2.0), h2o.H2O_ERR_INVALID),
    (dict(slot_format=1, k_scale=float("inf"), v_scale=1.0), h2o.H2O_ERR_INVALID),
    (dict(slot_format=1, k_scale=1.0, v_scale=float("nan")), h2o.H2O_ERR_INVALID),
])
def test_descriptor_checks(kw, status):
    d = desc(**kw)
    assert h2o.h2o_reset(d, 0) == status
    assert h2o.h2o_last_error() != ""
    assert h2o.h2o_decode_step(d, 5, A, A, A, A, None, 0, 0, 0) == status
    assert h2o.h2o_prefill(d, A, A, A, 8, A, 0, A, 1 << 20, 0) == status


def test_e4m3_slots_take_the_input_dtype_workspace():
    # E4M3 slots change the row bytes, not the launch plan: the workspace is the same.
    for dt in (h2o.H2O_F16, h2o.H2O_BF16):
        for kh in (4, 300, 3000):
            a = desc(dtype=dt, k_heavy=kh)
            b = desc(dtype=dt, k_heavy=kh, slot_format=1, k_scale=0.5, v_scale=2.0)
            for T in (0, 100, 1000):
                assert h2o.h2o_workspace_bytes(b, T) == h2o.h2o_workspace_bytes(a, T) > 0 or T == 0
    # scales are not read for slots in the input dtype
    assert h2o.h2o_workspace_bytes(desc(k_scale=0.0, v_scale=float("nan")), 16) > 0


def test_null_descriptor():
    lib = h2o.library()
    assert lib.h2o_reset(None, None) == h2o.H2O_ERR_INVALID
    assert lib.h2o_workspace_bytes(None, 4) == 0


@pytest.mark.parametrize("args,status", [
    (dict(T=-1), h2o.H2O_ERR_INVALID),
    (dict(q=0), h2o.H2O_ERR_INVALID),
    (dict(out=A + 4), h2o.H2O_ERR_INVALID),
    (dict(colsum=A + 2), h2o.H2O_ERR_INVALID),
    (dict(ws=0), h2o.H2O_ERR_WORKSPACE),
    (dict(ws_bytes=16), h2o.H2O_ERR_WORKSPACE),
    (dict(ws=A + 16), h2o.H2O_ERR_INVALID),
    # one unit's prompt rows past 2^31 - 1 bytes (2^23 + 1 rows of 128 fp16)
    (dict(T=2**23 + 1), h2o.H2O_ERR_UNSUPPORTED),
])
def test_prefill_checks(args, status):
    a = dict(q=A, k=A, v=A, T=64, out=A, colsum=0, ws=A, ws_bytes=1 << 20)
    a.update(args)
    st = h2o.h2o_prefill(desc(), a["q"], a["k"], a["v"], a["T"], a["out"], a["colsum"],
                         a["ws"], a["ws_bytes"], 0)
    assert st == status, h2o.h2o_last_error()


@pytest.mark.parametrize("args,status", [
    (dict(t=-1), h2o.H2O_ERR_INVALID),
    (dict(t=2**31 - 1), h2o.H2O_ERR_INVALID),
    (dict(t=2**40), h2o.H2O_ERR_INVALID),
    (dict(q=0), h2o.H2O_ERR_INVALID),
    (dict(k_new=A + 8), h2o.H2O_ERR_INVALID),
    (dict(aux=DecodeAux(A + 2, 0, 0)), h2o.H2O_ERR_INVALID),
])
def test_decode_checks(args, status):
    a = dict(t=10, q=A, k_new=A, v_new=A, out=A, aux=None)
    a.update(args)
    st = h2o.h2o_decode_step(desc(), a["t"], a["q"], a["k_new"], a["v_new"], a["out"], a["aux"],
                             0, 0, 0)
    assert st == status, h2o.h2o_last_error()


@pytest.mark.parametrize("args,status", [
    (dict(t=-1), h2o.H2O_ERR_INVALID),
    (dict(q=0), h2o.H2O_ERR_INVALID),
    (dict(out=A + 4), h2o.H2O_ERR_INVALID),
    (dict(aux=DecodeAux(0, 0, A + 1)), h2o.H2O_ERR_INVALID),
    (dict(desc=dict(k_local=0)), h2o.H2O_ERR_INVALID),
    (dict(desc=dict(head_dim=96)), h2o.H2O_ERR_UNSUPPORTED),
    # a split decode whose scratch exceeds the static array (8192 slots, 300 units of fp32)
    (dict(desc=dict(batch=100, heads=3, k_heavy=8000, k_local=192, dtype=h2o.H2O_F32)),
     h2o.H2O_ERR_UNSUPPORTED),
])
def test_decode_noalloc_checks(args, status):
    # Every check of h2o_decode_step, and the static scratch's limit, before any HIP call.
    a = dict(t=10, q=A, k_new=A, v_new=A, out=A, aux=None, desc={})
    a.update(args)
    st = h2o.h2o_decode_step_noalloc(desc(**a["desc"]), a["t"], a["q"], a["k_new"], a["v_new"],
                                     a["out"], a["aux"], 0)
    assert st == status, h2o.h2o_last_error()
    if status == h2o.H2O_ERR_UNSUPPORTED and "batch" in a["desc"]:
        need = h2o.h2o_workspace_bytes(desc(**a["desc"]), 0)
        assert need > h2o.H2O_NOALLOC_SCRATCH_BYTES
        assert "static scratch" in h2o.h2o_last_error()


@pytest.mark.parametrize("args,status", [
    (dict(lens=0), h2o.H2O_ERR_INVALID),
    (dict(lens=A + 2), h2o.H2O_ERR_INVALID),
    (dict(T=-1), h2o.H2O_ERR_INVALID),
    (dict(q=0), h2o.H2O_ERR_INVALID),
    (dict(ws=0), h2o.H2O_ERR_WORKSPACE),
    (dict(desc=dict(heads=0)), h2o.H2O_ERR_INVALID),
])
def test_prefill_ragged_checks(args, status):
    a = dict(q=A, k=A, v=A, T=64, lens=A, out=A, colsum=0, ws=A, ws_bytes=1 << 20, desc={})
    a.update(args)
    st = h2o.h2o_prefill_ragged(desc(**a["desc"]), a["q"], a["k"], a["v"], a["T"], a["lens"],
                                a["out"], a["colsum"], a["ws"], a["ws_bytes"], 0)
    assert st == status, h2o.h2o_last_error()


@pytest.mark.parametrize("args,status", [
    (dict(t=0), h2o.H2O_ERR_INVALID),
    (dict(t=A + 1), h2o.H2O_ERR_INVALID),
    (dict(q=0), h2o.H2O_ERR_INVALID),
    (dict(aux=DecodeAux(0, A + 2, 0)), h2o.H2O_ERR_INVALID),
    (dict(desc=dict(k_local=0)), h2o.H2O_ERR_INVALID),
])
def test_decode_ragged_checks(args, status):
    a = dict(t=A, q=A, k_new=A, v_new=A, out=A, aux=None, desc={})
    a.update(args)
    st = h2o.h2o_decode_step_ragged(desc(**a["desc"]), a["t"], a["q"], a["k_new"], a["v_new"],
                                    a["out"], a["aux"], 0, 0, 0)
    assert st == status, h2o.h2o_last_error()


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    import kv_cache_eviction_03_amd._abi as abi
    monkeypatch.setattr(abi, "_lib", None)
    monkeypatch.setattr(abi, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        abi.library()


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "h2o.h"

int main(void) {
  /* Fake device addresses: only host-side checks run, nothing is dereferenced. */
  static char slots[64];
  h2o_cache_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 8; d.heads = 32; d.head_dim = 128; d.k_heavy = 52; d.k_local = 52;
  d.dtype = H2O_F16; d.k_slots = slots; d.v_slots = slots + 16;
  d.slot_pos = (int32_t*)(void*)(slots + 32); d.acc_score = (float*)(void*)(slots + 48);
  d.policy = H2O_POLICY_H2O; d.slot_format = H2O_SLOTS_INPUT; d.k_scale = 1.0f; d.v_scale = 1.0f;
  printf("ws %zu\n", h2o_workspace_bytes(&d, 512));
  {
    h2o_status st = h2o_decode_step(&d, 512, NULL, slots, slots, (float*)(void*)slots, NULL,
                                    NULL, 0, NULL);
    printf("st %d %s\n", (int)st, h2o_status_str(st));
    printf("err %s\n", h2o_last_error());
  }
  d.k_local = 0;
  printf("desc %d\n", (int)h2o_reset(&d, NULL));
  return 0;
}
"""


def test_header_is_c99_and_links_from_c(tmp_path):
    # include/h2o.h is a plain C header: a C99 program compiles against it with warnings as
    # errors, links libh2o.so, and sees the same host-side results as the Python binding.
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi_check.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi_check"
    from kv_cache_eviction_03_amd._abi import LIB_PATH
    lib_dir = os.path.dirname(LIB_PATH)
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           f"-I{os.path.join(ROOT, 'include')}",
           str(src), "-o", str(exe), f"-L{lib_dir}", "-lh2o", f"-Wl,-rpath,{lib_dir}",
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    lines = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert int(lines["ws"]) == h2o.h2o_workspace_bytes(
        desc(batch=8, heads=32, k_heavy=52, k_local=52), 512) > 0
    st, name = lines["st"].split(" ", 1)
    assert int(st) == h2o.H2O_ERR_INVALID and name == h2o.h2o_status_str(h2o.H2O_ERR_INVALID)
    assert "NULL" in lines["err"]
    assert int(lines["desc"]) == h2o.H2O_ERR_INVALID
