"""Host-side accounting of the benchmark (no GPU): the algorithmic bytes and
credited FLOPs it divides by.  The expected values are the minimum-traffic and
work figures of the workloads written out by hand (Q, K, V read once, O and
one fp32 LSE per row written once; forward 4 N^2 d per head, halved when
causal, backward 10 N^2 d)."""

import dataclasses
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import fa_inputs as fi  # noqa: E402


def test_forward_bytes_single_head_fp32():
    # 3 x 256 x 64 x 4 bytes in, 256 x 64 x 4 out, 256 x 4 of LSE
    assert bench.forward_bytes(fi.CONFIGS[1]) == 3 * 65536 + 65536 + 1024 == 263168


def test_forward_bytes_bf16_workloads():
    per_head = 4 * 8192 * 128 * 2 + 8192 * 4
    assert bench.forward_bytes(fi.CONFIGS[3]) == 32 * per_head == 269484032
    assert bench.forward_bytes(fi.CONFIGS[5]) == 64 * per_head
    per_head_2k = 4 * 2048 * 128 * 2 + 2048 * 4
    assert bench.forward_bytes(fi.CONFIGS[2]) == 128 * per_head_2k == 269484032


def test_forward_bytes_fp8_and_other_key_count():
    cfg = dataclasses.replace(fi.CONFIGS[3], dtype="e4m3")
    # E4M3 Q, K, V; bf16 O; fp32 LSE
    assert bench.forward_bytes(cfg) == 32 * (3 * 8192 * 128 + 8192 * 128 * 2 + 8192 * 4)
    cfg = fi.CONFIGS[3]
    nk = 16384
    assert bench.forward_bytes(cfg, Nk=nk) == 32 * (8192 * 128 * 2 * 2 + 2 * nk * 128 * 2
                                                    + 8192 * 4)


def test_step_flops_training_step():
    cfg = fi.CONFIGS[5]
    per_head_fwd = 4 * 8192 * 8192 * 128 // 2
    per_head_bwd = 10 * 8192 * 8192 * 128 // 2
    assert bench.step_flops(cfg) == 64 * (per_head_fwd + per_head_bwd) == 3848290697216
