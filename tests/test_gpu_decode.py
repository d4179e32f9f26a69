"""Decode and merge parity on the GPU: fa_decode and fa_merge_states through
the C ABI against the fp64 oracle on the same seeded inputs.

Tolerances are the forward's: O max-abs <= 2e-2 for bf16 inputs, <= 5e-3 for
f16 and <= 1e-5 for fp32; LSE <= 1e-3 + 1e-5 |LSE| for the 16-bit formats and
<= 1e-5 for fp32; an empty cache must give O == 0 and LSE == -inf exactly.
"""

import dataclasses

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_helpers import check_lse, from_device, lib, log_case, max_abs, to_device, torch_cuda

pytestmark = pytest.mark.gpu

O_TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 5e-3}
LSE_TOL = {"f32": (1e-5, 0.0), "bf16": (1e-3, 1e-5), "f16": (1e-3, 1e-5)}


def run_decode(torch, cfg, inputs, stream=None):
    fa = lib()
    q, k, v = (to_device(torch, inputs[n], cfg.dtype) for n in ("q", "k", "v"))
    lens = inputs["lengths"]
    lens = None if lens is None else torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    if stream is None:
        o, lse = fa.decode(q, k, v, scale=cfg.scale, seqlens_k=lens)
    else:
        with torch.cuda.stream(stream):
            o, lse = fa.decode(q, k, v, scale=cfg.scale, seqlens_k=lens)
    torch.cuda.synchronize()
    return from_device(o, cfg.dtype), lse.cpu().numpy().astype(np.float64)


def check_decode(cfg, o, lse, ref_o, ref_lse):
    assert not np.any(np.isnan(o))
    err = max_abs(o, ref_o)
    assert err <= O_TOL[cfg.dtype], f"O max abs error {err:.3e}"
    check_lse(lse, ref_lse, *LSE_TOL[cfg.dtype])
    assert np.all(o[np.isneginf(ref_lse)] == 0.0)
    return err


def oracle_decode(cfg, inputs, heads=None):
    q, k, v = (fi.widen(inputs[n], cfg.dtype) for n in ("q", "k", "v"))
    lens = inputs["lengths"]
    if heads is None:
        return oracle.attention_decode(q, k, v, cfg.scale, lens)
    o = np.zeros((len(heads), cfg.d))
    lse = np.zeros(len(heads))
    for i, (b, h) in enumerate(heads):
        sub = None if lens is None else [lens[b]]
        ro, rl = oracle.attention_decode(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                         v[b:b + 1, h:h + 1], cfg.scale, sub)
        o[i], lse[i] = ro[0, 0], rl[0, 0]
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 96, 128, 192, 256])
@pytest.mark.parametrize("N,lengths", [
    (1, None), (63, None), (300, "zero_then_uniform"), (300, [300, 1, 0]), (5000, None),
    (5000, [4097, 4096, 64]), (9000, "zero_then_uniform"),
])
def test_decode_small_shapes(dtype, d, N, lengths):
    torch = torch_cuda()
    cfg = dataclasses.replace(fi.DECODE, B=3, H=2, N=N, d=d, dtype=dtype)
    log_case(test="decode_small", dtype=dtype, d=d, N=N, lengths=lengths)
    if isinstance(lengths, list):
        inputs = fi.make_decode_inputs(cfg, seed=5)
        inputs["lengths"] = np.array(lengths, np.int32)
    else:
        inputs = fi.make_decode_inputs(cfg, seed=5, lengths=lengths)
    o, lse = run_decode(torch, cfg, inputs)
    ref_o, ref_lse = oracle_decode(cfg, inputs)
    check_decode(cfg, o, lse, ref_o, ref_lse)


@pytest.mark.parametrize("lengths", [None, "zero_then_uniform"])
def test_decode_workload_sampled_heads(lengths):
    torch = torch_cuda()
    cfg = fi.DECODE
    log_case(test="decode_workload", shape=cfg.shape, lengths=lengths)
    inputs = fi.make_decode_inputs(cfg, seed=0, lengths=lengths)
    o, lse = run_decode(torch, cfg, inputs)
    rng = np.random.default_rng(9)
    heads = [(b, int(rng.integers(cfg.H))) for b in range(cfg.B)] + [(0, 0), (cfg.B - 1, cfg.H - 1)]
    ref_o, ref_lse = oracle_decode(cfg, inputs, heads)
    idx = tuple(np.array(heads).T)
    check_decode(cfg, o[idx], lse[idx], ref_o, ref_lse)
    if lengths is not None:
        # sequence 0 has an empty cache
        assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))


def test_decode_one_long_row_many_parts():
    torch = torch_cuda()
    cfg = dataclasses.replace(fi.DECODE, B=2, H=1, N=1 << 16)
    log_case(test="decode_long_row", shape=cfg.shape)
    inputs = fi.make_decode_inputs(cfg, seed=2)
    inputs["lengths"] = np.array([1 << 16, (1 << 16) - 1000], np.int32)
    o, lse = run_decode(torch, cfg, inputs)
    ref_o, ref_lse = oracle_decode(cfg, inputs)
    check_decode(cfg, o, lse, ref_o, ref_lse)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("parts,d", [(1, 128), (7, 64), (300, 128), (4096, 64), (5, 96), (33, 192)])
def test_merge_states_against_oracle(out_dtype, parts, d):
    torch = torch_cuda()
    fa = lib()
    log_case(test="merge", out_dtype=out_dtype, parts=parts, d=d)
    rng = np.random.default_rng([parts, d])
    R = 37
    o_parts = rng.standard_normal((R, parts, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((R, parts)) * 20.0).astype(np.float32)
    lse_parts[rng.random((R, parts)) < 0.3] = -np.inf
    lse_parts[3] = -np.inf                       # a row with every part empty
    lse_parts[5, 1:] = -np.inf                   # a row with one live part
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out_dtype]
    o, lse = fa.merge_states(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda(),
                             dtype=dt)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.merge_states(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    got = from_device(o, out_dtype)
    # fp32 arithmetic over `parts` terms, then the output rounding
    tol = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-5}[out_dtype]
    assert max_abs(got, ref_o) <= tol
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, 1e-5, 1e-6)
    assert np.all(got[3] == 0.0)


def test_decode_is_deterministic_and_stream_aware():
    torch = torch_cuda()
    cfg = dataclasses.replace(fi.DECODE, B=4, H=8, N=3000)
    log_case(test="decode_determinism", shape=cfg.shape)
    inputs = fi.make_decode_inputs(cfg, seed=3, lengths="zero_then_uniform")
    o1, l1 = run_decode(torch, cfg, inputs)
    o2, l2 = run_decode(torch, cfg, inputs, stream=torch.cuda.Stream())
    assert np.array_equal(o1, o2)
    assert np.array_equal(l1, l2)


def test_decode_at_the_part_limit():
    # one row of 2^20 keys: 4096 parts of 256 keys, the most a merge takes
    torch = torch_cuda()
    fa = lib()
    cfg = dataclasses.replace(fi.DECODE, B=1, H=1, N=1 << 20, d=64)
    parts = fa.fa_decode_workspace_size(fa.FA_DTYPE_BF16, 1, 1, cfg.N, 64) // (65 * 4)
    assert parts == 4096
    log_case(test="decode_part_limit", shape=cfg.shape, parts=parts)
    inputs = fi.make_decode_inputs(cfg, seed=8)
    inputs["lengths"] = np.array([(1 << 20) - 5], np.int32)
    o, lse = run_decode(torch, cfg, inputs)
    ref_o, ref_lse = oracle_decode(cfg, inputs)
    check_decode(cfg, o, lse, ref_o, ref_lse)
