"""Seeded synthetic inputs and workload accounting for the attention path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no attention arithmetic: it draws seeded normal tensors, rounds them
to bf16 bit patterns, defines the five workloads and counts their credited
FLOPs and minimum bytes.

Workloads (all tensors [B, H, N, d], contiguous, entries iid N(0, 1)):
  1  single head, N=256, d=64, fp32, non-causal, scale 1/8
  2  B=4, H=32, N=2048, d=128, bf16, non-causal
  3  B=1, H=32, N=8192, d=128, bf16, causal
  4  B=8, H=32, padded N=32768, d=128, bf16, causal + per-sequence key
     lengths (sequence 0 has length 0; the rest uniform in [1, N]);
     Q drawn x30 before rounding so raw scores reach about +-90
  5  B=2, H=32, N=8192, d=128, bf16, causal, forward + backward with dO

The 8,192-token, d=128, 32-head shape is the running example of the source
pages ("What is FlashAttention?" Step 1; "FlashAttention" byte-accounting
panel; "Explain FlashAttention and why it is IO-aware", byte arithmetic);
these seeded tensors stand in for real activations.

Random streams: numpy default_rng([seed, tensor_id, b, h]) (PCG64 seeded via
SeedSequence) with tensor_id Q=0, K=1, V=2, dO=3; lengths use
default_rng([seed, 4]).  Draws are float32 standard normals; bf16 tensors
are rounded to nearest-even from them.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "Config", "CONFIGS", "TENSOR_IDS",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "f32_to_f16_bits", "HALF_DTYPES", "widen",
    "make_lengths", "make_head", "make_tensor", "make_inputs",
    "packed_lengths", "offsets", "make_packed",
    "E4M3_MAX", "e4m3_bits_to_f64", "f64_to_e4m3_bits", "FP8_DESCALE", "storage_dtype",
    "credited_flops", "useful_pairs", "useful_flops", "min_bytes",
]

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "lengths": 4}


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32", "bf16" or "f16"
    causal: bool
    lengths: str | None   # None, or "zero_then_uniform"
    q_mult: float = 1.0
    backward: bool = False

    @property
    def scale(self) -> float:
        """fp32 value of 1/sqrt(d), the scale every workload uses."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


CONFIGS = {
    1: Config(1, "single-head N=256 d=64 fp32 non-causal", 1, 1, 256, 64, "f32", False, None),
    2: Config(2, "B=4 H=32 N=2048 d=128 bf16 non-causal", 4, 32, 2048, 128, "bf16", False, None),
    3: Config(3, "B=1 H=32 N=8192 d=128 bf16 causal", 1, 32, 8192, 128, "bf16", True, None),
    4: Config(4, "B=8 H=32 N=32768 d=128 bf16 causal+key-lengths Qx30", 8, 32, 32768, 128,
              "bf16", True, "zero_then_uniform", q_mult=30.0),
    5: Config(5, "B=2 H=32 N=8192 d=128 bf16 causal fwd+bwd", 2, 32, 8192, 128, "bf16",
              True, None, backward=True),
}


# ---------------------------------------------------------------------------
# bf16 bit patterns
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits.

    NaN stays NaN (quiet); infinities and overflow to infinity follow IEEE
    rounding.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
               >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16),
                           rounded)
    return rounded


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


HALF_DTYPES = ("bf16", "f16")

# FP8 workloads store E4M3 codes of x / descale, x the same N(0,1) draws as
# the other formats; the powers of two keep |x| / descale (|x| <= ~5.5) under
# 448 and make dequantisation exact.  O (the dequantised V times softmax) and
# dO stay bf16.
FP8_DESCALE = {"q": 2.0 ** -4, "k": 2.0 ** -5, "v": 2.0 ** -6}


def storage_dtype(dtype):
    """NumPy storage of a device format: bf16 / f16 bits, E4M3 codes, fp32."""
    return {"bf16": np.uint16, "f16": np.uint16, "e4m3": np.uint8}.get(dtype, np.float32)


def f32_to_f16_bits(x):
    """Round float32 values to IEEE binary16 (nearest, ties to even); uint16 bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


E4M3_MAX = 448.0


def e4m3_bits_to_f64(bits):
    """Exact values of OCP FP8 E4M3 codes (uint8): sign, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); no
    infinities; S.1111.111 is NaN, so the largest finite value is 448."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def f64_to_e4m3_bits(x):
    """Round values to OCP FP8 E4M3 (nearest, ties to even) and return the
    uint8 codes.  Values whose rounding exceeds 448 in magnitude, and NaN,
    raise ValueError: the generators never produce them."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("NaN has no E4M3 encoding here")
    a = np.abs(x)
    # quantum of the binade: 2^(e - 3) for normals (e >= -6), 2^-9 below
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    q = np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int64))
    r = np.round(a / q) * q                      # numpy rounds halves to even
    if np.any(r > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    e_r = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, e_r + 7, 0).astype(np.int64)
    mant = np.where(normal, r / np.ldexp(1.0, e_r.astype(np.int64)) * 8 - 8, r / 2.0 ** -9)
    code = (exp_field << 3) | np.rint(mant).astype(np.int64)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def widen(arr, dtype):
    """Exact float64 values of a device-format array (fp32, or bf16 / f16 /
    E4M3 codes)."""
    if dtype == "e4m3":
        return e4m3_bits_to_f64(arr)
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(arr, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Seeded generation
# ---------------------------------------------------------------------------

def make_lengths(cfg: Config, seed: int = 0):
    """Per-sequence key lengths (int32 [B]) or None."""
    if cfg.lengths is None:
        return None
    if cfg.lengths != "zero_then_uniform":
        raise ValueError(f"unknown lengths recipe {cfg.lengths!r}")
    rng = np.random.default_rng([seed, TENSOR_IDS["lengths"]])
    rest = rng.integers(1, cfg.N, endpoint=True, size=cfg.B - 1)
    return np.concatenate([[0], rest]).astype(np.int32)


def make_head(cfg: Config, name: str, b: int, h: int, seed: int = 0, N: int | None = None,
              d: int | None = None):
    """One head's [N, d] tensor in device format (float32, or bf16 / f16 bits)."""
    N = cfg.N if N is None else N
    d = cfg.d if d is None else d
    rng = np.random.default_rng([seed, TENSOR_IDS[name], b, h])
    x = rng.standard_normal(N * d, dtype=np.float32).reshape(N, d)
    if name == "q" and cfg.q_mult != 1.0:
        x = x * np.float32(cfg.q_mult)
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(x)
    if cfg.dtype == "f16":
        return f32_to_f16_bits(x)
    if cfg.dtype == "e4m3":
        return f64_to_e4m3_bits(x.astype(np.float64) / FP8_DESCALE[name])
    return x


def make_tensor(cfg: Config, name: str, seed: int = 0, threads: int | None = None,
                B: int | None = None, H: int | None = None, N: int | None = None,
                d: int | None = None):
    """Full [B, H, N, d] tensor in device format, built head by head.

    Heads are drawn in parallel threads (numpy releases the GIL while it
    fills arrays); the result does not depend on the thread count.
    """
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    N = cfg.N if N is None else N
    d = cfg.d if d is None else d
    out = np.empty((B, H, N, d), storage_dtype(cfg.dtype))

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = make_head(cfg, name, b, h, seed, N, d)

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or B * H == 1:
        for bh in range(B * H):
            fill(bh)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(B * H)))
    return out


def make_inputs(cfg: Config, seed: int = 0, with_grad: bool | None = None, **shape_overrides):
    """Dict of device-format host arrays for a workload: q, k, v (and do),
    lengths (int32 [B] or None) and scale (float)."""
    with_grad = cfg.backward if with_grad is None else with_grad
    names = ["q", "k", "v"] + (["do"] if with_grad else [])
    res = {n: make_tensor(cfg, n, seed, **shape_overrides) for n in names}
    res["lengths"] = make_lengths(cfg, seed)
    res["scale"] = cfg.scale
    return res


def packed_lengths(B: int, max_len: int, seed: int = 0, empty_first: bool = True):
    """Sequence lengths of a packed batch (int32 [B]): uniform in
    [1, max_len], the first one 0 when ``empty_first`` (an empty sequence),
    and one of them max_len so the longest sequence is present."""
    rng = np.random.default_rng([seed, TENSOR_IDS["lengths"], 1])
    lens = rng.integers(1, max_len, endpoint=True, size=B)
    if B > 1:
        lens[rng.integers(1 if empty_first else 0, B)] = max_len
    if empty_first and B > 0:
        lens[0] = 0
    return lens.astype(np.int32)


def offsets(lengths):
    """Cumulative offsets (int32 [B + 1]) of packed sequences."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


def make_packed(cfg: Config, name: str, lengths, seed: int = 0, H: int | None = None,
                d: int | None = None):
    """Packed head-major [H, sum(lengths), d] tensor in device format:
    sequence b's rows of head h are make_head(cfg, name, b, h) with
    lengths[b] rows, placed back to back."""
    H = cfg.H if H is None else H
    d = cfg.d if d is None else d
    lengths = [int(n) for n in lengths]
    out = np.empty((H, sum(lengths), d), storage_dtype(cfg.dtype))
    start = 0
    for b, n in enumerate(lengths):
        for h in range(H):
            out[h, start:start + n] = make_head(cfg, name, b, h, seed, n, d)
        start += n
    return out


# ---------------------------------------------------------------------------
# Work accounting
# ---------------------------------------------------------------------------

def credited_flops(B, H, N, d, causal, backward=False):
    """FLOPs credited to one call.

    Forward: 4 N^2 d per head, halved for a causal model, the throughput
    convention of "FlashAttention" (deepconcepts.dev), "Checking it on a real
    system".  Backward: 10 N^2 d per head (five N x N x d contractions: the S
    recompute, dP, dV, dK and dQ), halved when causal.
    """
    per_head = (10 if backward else 4) * N * N * d
    total = per_head * B * H
    return total // 2 if causal else total


def useful_pairs(N, causal, lengths=None, B=1, Nk=None):
    """Visible (query, key) pairs per head, summed over the batch: N query
    rows, Nk keys (default N), key length L (clamped to [0, Nk]); with the
    causal mask row i sees min(L, max(0, i + Nk - N + 1)) keys, without it L."""
    Nk = N if Nk is None else Nk
    rows = np.arange(N, dtype=np.int64)
    total = 0
    for b in range(B):
        L = Nk if lengths is None else int(min(max(int(lengths[b]), 0), Nk))
        if causal:
            total += int(np.clip(rows + (Nk - N) + 1, 0, L).sum())
        else:
            total += N * L
    return total


def useful_flops(B, H, N, d, causal, lengths=None, backward=False, Nk=None):
    """FLOPs on visible pairs only: 4d (forward) or 10d (backward) per pair."""
    return (10 if backward else 4) * d * H * useful_pairs(N, causal, lengths, B, Nk)


def min_bytes(B, H, N, d, es, backward=False):
    """Minimum HBM bytes: every input read once, every output written once.

    Forward: Q, K, V read and O written (es bytes each) plus one fp32 LSE per
    row.  Backward: Q, K, V, O, dO read, dQ, dK, dV written, LSE read and the
    fp32 row dot products D written and read once.
    """
    nd = B * H * N * d
    rows = B * H * N
    if not backward:
        return 4 * nd * es + 4 * rows
    return 8 * nd * es + 4 * rows + 8 * rows


# ---------------------------------------------------------------------------
# Decoding against a cache
# ---------------------------------------------------------------------------

# One new query row per (batch, head) against a cache shaped like the pages'
# running example (8,192 positions, d = 128, 32 heads), batch 8.
DECODE = Config(0, "decode: B=8 H=32 cache 8192 d=128 bf16", 8, 32, 8192, 128, "bf16", False,
                None)


def make_decode_inputs(cfg: Config, seed: int = 0, lengths: str | None = None):
    """q [B, H, d] (row 0 of each head's q stream), k and v [B, H, N, d]
    caches in device format, and int32 [B] cached lengths (None = all N;
    "zero_then_uniform" as for the forward workloads)."""
    q = make_tensor(cfg, "q", seed, N=1)[:, :, 0]
    k = make_tensor(cfg, "k", seed)
    v = make_tensor(cfg, "v", seed)
    lens = None
    if lengths is not None:
        lens = make_lengths(dataclasses.replace(cfg, lengths=lengths), seed)
    return {"q": np.ascontiguousarray(q), "k": k, "v": v, "lengths": lens}


def decode_bytes(B, H, N, d, es, lengths=None):
    """Minimum HBM bytes of a decode step: the visible cache rows of K and V
    read once, q read and o written once, one fp32 LSE per row."""
    if lengths is None:
        cached = B * N
    else:
        cached = int(np.clip(np.asarray(lengths, np.int64), 0, N).sum())
    return H * (2 * cached * d * es) + B * H * (2 * d * es + 4)
