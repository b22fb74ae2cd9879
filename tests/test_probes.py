"""The measurement probes (libh2o_probes.so): exported symbols, host-side argument checks
(no GPU call is made when they fail) and the LDS probe's address patterns."""
import ctypes
import os

import pytest

import bench

from kv_cache_eviction_03_amd.build import PROBE_LIB


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libh2o_probes.so is not built")
    return bench._probe_lib()


def test_probe_library_exports(lib):
    for name in ("hbm_read_probe", "mfma_probe", "mfma_probe_flops", "lds_bank_probe",
                 "issue_overlap_probe"):
        assert hasattr(lib, name), name


def test_lds_probe_rejects_bad_offsets_before_any_gpu_call(lib):
    # -1 is returned by the host checks, ahead of any HIP call (there is no GPU here)
    good = [l * 16 for l in range(64)]
    for mode, offs in ((0, [8] + good[1:]),               # not 16-byte aligned for b128
                       (0, [65536 - 8] + good[1:]),       # runs past the 64 KB array
                       (1, [-16] + good[1:]),             # negative (only -1 means idle)
                       (4, good),                         # no such mode
                       (3, [4] + good[1:])):              # not 8-byte aligned for b64
        arr = (ctypes.c_int * 64)(*offs)
        assert lib.lds_bank_probe(arr, None, mode, 10, None, None) == -1, (mode, offs[0])
    arr = (ctypes.c_int * 64)(*good)
    assert lib.lds_bank_probe(arr, None, 0, 0, None, None) == -1    # iters < 1


def test_lds_patterns_are_in_bounds():
    pats = bench._lds_patterns()
    assert len({p[0] for p in pats}) == len(pats)                   # names identify dispatches
    for name, mode, offs in pats:
        size = 16 if mode == 0 else 8
        assert len(offs) == 64, name
        assert all(o == -1 or (0 <= o and o % size == 0 and o + size <= 65536) for o in offs), name
        assert any(o >= 0 for o in offs), name


def test_overlap_probe_rejects_bad_arguments_before_any_gpu_call(lib):
    # mode, waves per SIMD, workgroups, iterations: each out of range returns -1 unlaunched
    for args in ((-1, 1, 256, 10), (len(bench.OVERLAP_MODES), 1, 256, 10), (0, 0, 256, 10),
                 (0, 3, 256, 10), (0, 1, 0, 10), (0, 1, 256, 0)):
        assert lib.issue_overlap_probe(*args, None, None, None) == -1, args
    assert sorted(bench.OVERLAP_MODES) == list(range(len(bench.OVERLAP_MODES)))
