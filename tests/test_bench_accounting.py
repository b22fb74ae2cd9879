"""The algorithmic work bench.py divides by kernel time (its roofline numerators), pinned to
values worked out by hand from the per-unit formulas:

  decode, bytes per unit-step = 2·k·d·s_slot (K and V slot rows) + 12·k (positions read,
      scores read and written) + 3·d·s (q, k_new, v_new) + 4·d (fp32 output)
      + 2·d·s_slot (the new row written) + 8 (its position and score);
  prefill, flops per unit = 2·T·(T + 1)·d (causal QK^T and PV, diagonal included);
  prefill, bytes per unit = 3·T·d·s + 4·T·d + 4·T + 2·k·d·s + 8·k.

s is the input element size; s_slot is s, or 1 for E4M3 slots.
"""
import bench
from workloads import WORKLOADS


def test_decode_bytes_per_unit_step():
    # tiny fp32 (d 64, k 32): 16384 + 384 + 768 + 256 + 512 + 8
    assert bench.decode_bytes_per_unit(WORKLOADS[1]) == 18_312
    # OPT-6.7B layer fp16 (d 128, k 104): 53248 + 1248 + 768 + 512 + 512 + 8
    assert bench.decode_bytes_per_unit(WORKLOADS[2]) == 56_296
    assert bench.decode_bytes_per_unit(WORKLOADS[3]) == 56_296            # LLaMA-7B, bf16
    # OPT-30B layer fp16 (k 410): 209920 + 4920 + 768 + 512 + 512 + 8
    assert bench.decode_bytes_per_unit(WORKLOADS[4]) == 216_640
    # the 4096-slot stream, bf16: 2097152 + 49152 + 768 + 512 + 512 + 8
    assert bench.decode_bytes_per_unit(WORKLOADS[5]) == 2_148_104
    # one launch of the OPT-6.7B layer moves 256 units' worth
    assert bench.decode_bytes_per_unit(WORKLOADS[2]) * WORKLOADS[2].units_per_layer == 14_411_776
    # one launch of a LLaMA-7B layer (the headline's decode kernel) moves 2048 units' worth,
    # a model step 32 launches
    w = WORKLOADS[3]
    assert bench.decode_bytes_per_unit(w) * w.units_per_layer == 115_294_208
    assert bench.decode_bytes_per_unit(w) * w.units_per_layer * w.layers == 3_689_414_656


def test_decode_bytes_with_e4m3_slots():
    # slot rows one byte per element, q / k_new / v_new still fp16: 26624 + 1248 + 768 + 512
    # + 256 + 8
    w = WORKLOADS[2].scaled(slot_format="e4m3")
    assert bench.decode_bytes_per_unit(w) == 29_416
    assert bench.decode_bytes_per_unit(w) * w.units_per_layer == 7_530_496
    # the stream: 1048576 + 49152 + 768 + 512 + 256 + 8
    assert bench.decode_bytes_per_unit(WORKLOADS[5].scaled(slot_format="e4m3")) == 1_099_272


def test_prefill_work_per_unit():
    w = WORKLOADS[2]                                  # T 512, d 128, fp16, k 104
    assert bench.prefill_flops_per_unit(w) == 67_239_936
    # 393216 + 262144 + 2048 + 53248 + 832
    assert bench.prefill_bytes_per_unit(w) == 711_488
    w = WORKLOADS[4]                                  # T 2048, k 410: the MFMA-bound prompt
    assert bench.prefill_flops_per_unit(w) == 2 * 2048 * 2049 * 128
    assert bench.prefill_flops_per_unit(w) * w.units_per_layer == 962_542_436_352           # 962.5 GFLOP
    # arithmetic intensity above the 312.5 flop/B ridge of 2.5 PFLOP/s over 8 TB/s
    assert bench.prefill_flops_per_unit(w) / bench.prefill_bytes_per_unit(w) > 312.5
    assert bench.prefill_flops_per_unit(WORKLOADS[2]) / bench.prefill_bytes_per_unit(WORKLOADS[2]) < 312.5
    # the headline's 32-layer prefill: 2048 units per layer
    w = WORKLOADS[3]
    assert bench.prefill_flops_per_unit(w) * w.units_per_layer * w.layers == 4_406_636_445_696          # 67,239,936 x 65,536
