"""Parity on the GPU for the FP8 forward: E4M3 codes with per-tensor descale
factors, against the fp64 oracle on the dequantised inputs (code * descale).

The kernel rounds each key tile's probabilities to E4M3 for the second
product, so the bound is derived from that rounding (reading 11e): with
P_ij = exp(s_ij - LSE_i) on visible pairs,
    |O_i - O_i^ref| <= (2^-4 + 3 ds_i) sum_j P_ij |v_j|
                       + 2^-18 sum_j |v_j| + 2^-8 |O_i^ref| + 1e-6,
    |LSE_i - LSE_i^ref| <= ds_i + 1e-5 (1 + |LSE_i^ref|),
where 2^-4 is the relative rounding error of an E4M3 normal, 2^-18 the
absolute error of a probability below the normal range after the 2^8
scaling, 2^-8 covers the bf16 output, and ds_i = 2^-10 scale max_j
sum_t |q_it k_jt| bounds the error of the FP8 dot products (measured at most
2^-11.8 of the largest product).  Rows that see no key give O == 0 and
LSE == -inf exactly.
"""

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_helpers import custom, from_device, lib, log_case, torch_cuda

pytestmark = pytest.mark.gpu


def fp8_case(B, H, Nq, Nk, seed):
    cfg = custom(3, B=B, H=H, N=Nq, dtype="e4m3")
    codes = {n: fi.make_tensor(cfg, n, seed, N=(Nq if n == "q" else Nk)) for n in "qkv"}
    real = {n: fi.widen(codes[n], "e4m3") * fi.FP8_DESCALE[n] for n in "qkv"}
    return cfg, codes, real


def run_fp8(torch, codes, scale, causal, lengths):
    fa = lib()
    dev = {n: torch.from_numpy(np.ascontiguousarray(codes[n])).cuda() for n in codes}
    lens = None if lengths is None else torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    o, lse = fa.forward_fp8(dev["q"], dev["k"], dev["v"], fi.FP8_DESCALE["q"],
                            fi.FP8_DESCALE["k"], fi.FP8_DESCALE["v"], scale=scale, causal=causal,
                            seqlens_k=lens)
    torch.cuda.synchronize()
    return from_device(o, "bf16"), lse.cpu().numpy().astype(np.float64)


def bounds(q, k, v, rows, scale, causal, length, ref_o):
    """Per-row bounds of one head (q [rows], k, v [Nk, d])."""
    offset = k.shape[0] - q.shape[0]
    vis = oracle.visible_mask(rows, k.shape[0], causal, length, offset=offset)
    qa = np.abs(q[rows]) @ np.abs(k).T
    ds = 2.0 ** -10 * scale * np.max(np.where(vis, qa, 0.0), axis=1, initial=0.0)
    pv, _ = oracle.attention_rows(q, k, np.abs(v), rows, scale, causal, length)
    vsum = np.sum(np.where(vis[:, :, None], np.abs(v)[None], 0.0), axis=1)
    ob = ((2.0 ** -4 + 3 * ds)[:, None] * pv + 2.0 ** -18 * vsum + 2.0 ** -8 * np.abs(ref_o)
          + 1e-6)
    return ob, ds


def check_head(got_o, got_l, q, k, v, rows, scale, causal, length):
    ref_o, ref_l = oracle.attention_rows(q, k, v, rows, scale, causal, length)
    ob, ds = bounds(q, k, v, rows, scale, causal, length, ref_o)
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty), "empty-row LSE must be exactly -inf"
    assert np.all(got_o[empty] == 0.0)
    err = np.abs(got_o - ref_o)
    assert np.all(err <= ob), f"O err {err.max():.3e} (bound at worst row {ob.min():.3e})"
    fin = ~empty
    assert np.all(np.abs(got_l[fin] - ref_l[fin]) <= ds[fin] + 1e-5 * (1 + np.abs(ref_l[fin])))
    return err.max(), float(np.sqrt(np.mean(err ** 2))) if err.size else 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_against_the_oracle(causal):
    torch = torch_cuda()
    for Nq, Nk, lens in ((300, 300, None), (257, 257, [0, 1, 257, 200]), (64, 300, None),
                         (300, 100, None), (1, 512, None), (129, 129, [5, 129])):
        B = 2 if lens is None else len(lens)
        log_case(test="fp8", causal=causal, Nq=Nq, Nk=Nk, lengths=lens)
        cfg, codes, real = fp8_case(B, 2, Nq, Nk, seed=Nq + 7 * Nk)
        got_o, got_l = run_fp8(torch, codes, cfg.scale, causal, lens)
        worst = 0.0
        for b in range(B):
            length = None if lens is None else lens[b]
            for h in range(2):
                rows = np.arange(Nq)
                e, _ = check_head(got_o[b, h], got_l[b, h], real["q"][b, h], real["k"][b, h],
                                  real["v"][b, h], rows, cfg.scale, causal, length)
                worst = max(worst, e)
        print(f"max |O err| {worst:.3e}", flush=True)


def test_fp8_forward_sampled_rows_at_the_benchmark_shape():
    """B=1, H=32, N=8192, d=128, causal (the forward workload in FP8): rows
    sampled in every head against the oracle, one row at a time."""
    torch = torch_cuda()
    log_case(test="fp8-sampled", N=8192)
    cfg, codes, real = fp8_case(1, 32, 8192, 8192, seed=0)
    got_o, got_l = run_fp8(torch, codes, cfg.scale, True, None)
    rng = np.random.default_rng(5)
    for h in range(32):
        rows = np.unique(np.concatenate([[0, 8191], rng.integers(0, 8192, 6)]))
        check_head(got_o[0, h, rows], got_l[0, h, rows], real["q"][0, h], real["k"][0, h],
                   real["v"][0, h], rows, cfg.scale, True, None)
