"""Seeded generator, bf16 rounding and work accounting (CPU only)."""

import dataclasses
import json
import math
import os

import numpy as np
import pytest

import fa_inputs as fi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_generator_is_deterministic_and_thread_independent():
    cfg = fi.CONFIGS[2]
    a = fi.make_tensor(cfg, "q", B=2, H=3, N=64, threads=1)
    b = fi.make_tensor(cfg, "q", B=2, H=3, N=64, threads=4)
    assert a.dtype == np.uint16 and a.shape == (2, 3, 64, 128)
    assert np.array_equal(a, b)
    c = fi.make_tensor(cfg, "k", B=2, H=3, N=64, threads=1)
    assert not np.array_equal(a, c)
    # per-(b, h) streams: a head does not depend on the batch/head count
    d = fi.make_tensor(cfg, "q", B=3, H=5, N=64, threads=2)
    assert np.array_equal(a[1, 2], d[1, 2])
    assert np.array_equal(fi.make_head(cfg, "q", 1, 2, N=64), a[1, 2])


def test_generator_moments():
    cfg = fi.CONFIGS[3]
    x = fi.widen(fi.make_head(cfg, "v", 0, 7, N=4096), "bf16")
    assert abs(x.mean()) < 0.01
    assert abs(x.std() - 1.0) < 0.01
    f = fi.make_head(fi.CONFIGS[1], "q", 0, 0)
    assert f.dtype == np.float32 and f.shape == (256, 64)
    assert abs(f.astype(np.float64).std() - 1.0) < 0.02


def test_q_times_30_before_rounding():
    cfg = fi.CONFIGS[4]
    raw = np.random.default_rng([0, 0, 1, 3]).standard_normal(64 * 128, dtype=np.float32)
    expect = fi.f32_to_bf16_bits((raw * np.float32(30.0)).reshape(64, 128))
    assert np.array_equal(fi.make_head(cfg, "q", 1, 3, N=64), expect)
    # K and V are not scaled
    rawk = np.random.default_rng([0, 1, 1, 3]).standard_normal(64 * 128, dtype=np.float32)
    assert np.array_equal(fi.make_head(cfg, "k", 1, 3, N=64),
                          fi.f32_to_bf16_bits(rawk.reshape(64, 128)))


def test_lengths_recipe():
    cfg = fi.CONFIGS[4]
    L = fi.make_lengths(cfg)
    assert L.dtype == np.int32 and L.shape == (8,)
    assert L[0] == 0
    assert np.all((L[1:] >= 1) & (L[1:] <= cfg.N))
    assert np.array_equal(L, fi.make_lengths(cfg))
    assert fi.make_lengths(fi.CONFIGS[3]) is None


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(7.0),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, -1e-40,
                  1.00390625, 1.01171875, 1.0078125 + 2 ** -10], np.float32),
        # exact ties between two bf16 values (round to even both ways)
        (np.arange(1, 200, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32),
    ])
    ours = fi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan_bits = fi.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(fi.bf16_bits_to_f32(nan_bits)[0])


def test_bf16_widening_is_exact_round_trip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = fi.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(fi.f32_to_bf16_bits(f[finite]), bits[finite])
    assert np.array_equal(fi.widen(bits[finite], "bf16"), f[finite].astype(np.float64))


def test_scale_is_fp32_inverse_sqrt_d():
    assert fi.CONFIGS[1].scale == 0.125
    assert fi.CONFIGS[2].scale == float(np.float32(1 / math.sqrt(128)))


# ---------------------------------------------------------------------------
# Accounting pinned to the pages' printed arithmetic
# ---------------------------------------------------------------------------

def test_credited_flops_match_page_byte_arithmetic():
    g = golden("byte_accounting.json")
    f = fi.credited_flops(1, 1, g["N"], g["d"], causal=False)
    assert f == 4 * g["N"] ** 2 * g["d"]
    assert round(f / 1e9, 2) == g["two_products_gflop"]
    assert fi.credited_flops(1, 1, g["N"], g["d"], causal=True) == f // 2
    assert fi.credited_flops(2, 32, 8192, 128, True, backward=True) == 2 * 32 * 10 * 8192 ** 2 * 128 // 2


def test_min_bytes_match_page_minimum():
    g = golden("byte_accounting.json")
    N, d, es = g["N"], g["d"], g["element_bytes"]
    lse_bytes = 4 * N
    assert fi.min_bytes(1, 1, N, d, es) - lse_bytes == g["qkvo_minimum_bytes"]
    score_traffic = 4 * N * N * es
    assert score_traffic == g["score_transfers_bytes"]
    total = score_traffic + g["qkvo_minimum_bytes"]
    assert total == g["materialising_total_bytes"]
    assert total / 2 ** 20 == g["materialising_total_mib"]
    assert total / g["qkvo_minimum_bytes"] == g["ratio_to_minimum"]
    assert round(total / g["illustrative_bandwidth_bytes_per_s"] * 1e3, 3) == g["bandwidth_floor_ms"]
    assert N * N == g["score_matrix_elements"]
    assert N * es / 1024 == g["score_row_kib"]


def test_statistics_size_reading_one_fp32_per_row():
    """The panel's 65.0 MiB (and 260 MiB at 32,768 tokens) is the output plus
    ONE fp32 per row; the first page's 65,536 B per head is m and l (two)."""
    g = golden("memory_figures.json")
    p = g["panel"]
    H, N, d, es = p["heads"], p["N"], p["d"], p["element_bytes"]
    out = H * N * d * es
    lse = H * N * 4
    assert (out + lse) / 2 ** 20 == p["flash_peak_intermediate_mib"]
    N2 = 32768
    assert (H * N2 * d * es + H * N2 * 4) / 2 ** 20 == p["at_N_32768"]["flash_mib"]
    assert H * N * N * es / 2 ** 30 == p["standard_peak_intermediate_gib"]
    assert H * N2 * N2 * es / 2 ** 30 == p["at_N_32768"]["standard_gib"]
    assert 2 * 4 * 8192 == g["m_and_l_bytes_per_head_8192_fp32"]
    assert 8192 ** 2 * 2 / 2 ** 20 == g["score_matrix_one_head_8192_fp16_mib"]
    assert 32 * 8192 ** 2 * 2 / 2 ** 30 == g["score_matrices_32_heads_8192_fp16_gib"]
    assert 131072 ** 2 * 2 / 2 ** 30 == g["score_matrix_one_head_131072_fp16_gib"]
    assert (4 * 8192) ** 2 / 8192 ** 2 == g["growth_per_4x_tokens"]


def test_useful_pairs_brute_force():
    for N in (1, 2, 7, 16):
        for causal in (False, True):
            for L in range(0, N + 1):
                vis = oracle.visible_mask(np.arange(N), N, causal, L)
                assert fi.useful_pairs(N, causal, np.array([L])) == int(vis.sum())
    assert fi.useful_pairs(8, True) == 36
    assert fi.useful_flops(1, 2, 8, 4, True) == 4 * 4 * 2 * 36


def test_f16_rounding_matches_binary16_facts():
    """IEEE binary16: 1 = 0x3C00, 65504 = 0x7BFF (largest finite), 2^-24 =
    0x0001 (smallest subnormal); 1 + 2^-11 is a tie between 1 and 1 + 2^-10
    and rounds to the even 1; 1 + 3 * 2^-11 rounds up to 1 + 2^-9; 65520 rounds
    to infinity (0x7C00)."""
    x = np.array([1.0, 65504.0, 2.0 ** -24, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65520.0, -2.0],
                 np.float32)
    bits = fi.f32_to_f16_bits(x)
    assert bits.tolist() == [0x3C00, 0x7BFF, 0x0001, 0x3C00, 0x3C02, 0x7C00, 0xC000]
    w = fi.widen(bits, "f16")
    assert w.tolist()[:5] == [1.0, 65504.0, 2.0 ** -24, 1.0, 1 + 2.0 ** -9]


def test_f16_tensors_are_the_rounded_float32_draws():
    cfg = fi.CONFIGS[2]
    import dataclasses
    c16 = dataclasses.replace(cfg, dtype="f16", N=64)
    c32 = dataclasses.replace(cfg, dtype="f32", N=64)
    a = fi.widen(fi.make_head(c16, "k", 1, 3), "f16")
    b = fi.make_head(c32, "k", 1, 3).astype(np.float64)
    # the f16 value is the nearest binary16 value: within half an ulp
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(b), 2.0 ** -14))) - 10)
    assert np.all(np.abs(a - b) <= ulp / 2)


def test_useful_pairs_rectangular_brute_force():
    for N, Nk in ((5, 9), (9, 5), (1, 7), (7, 1), (6, 6)):
        for causal in (False, True):
            for L in (None, 0, 1, 3, Nk):
                lens = None if L is None else np.array([L])
                vis = oracle.visible_mask(np.arange(N), Nk, causal, L, offset=Nk - N)
                assert fi.useful_pairs(N, causal, lens, Nk=Nk) == int(vis.sum())


def test_packed_generators():
    lens = fi.packed_lengths(7, 300, seed=4)
    assert lens.dtype == np.int32 and lens[0] == 0 and lens.max() == 300
    assert np.all(lens[1:] >= 1) and np.all(lens <= 300)
    assert np.array_equal(fi.packed_lengths(7, 300, seed=4), lens)
    cu = fi.offsets(lens)
    assert cu.dtype == np.int32 and cu[0] == 0 and np.all(np.diff(cu) == lens)
    cfg = fi.CONFIGS[5]
    t = fi.make_packed(cfg, "k", [3, 0, 5], seed=2, H=2, d=64)
    assert t.shape == (2, 8, 64) and t.dtype == np.uint16
    assert np.array_equal(t[1, 3:8], fi.make_head(cfg, "k", 2, 1, 2, 5, 64))
    assert np.array_equal(t[0, 0:3], fi.make_head(cfg, "k", 0, 0, 2, 3, 64))


def test_e4m3_decoding_follows_the_format():
    """OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormals m * 2^-9, no
    infinities, S.1111.111 NaN; every code agrees with torch's float8_e4m3fn."""
    torch = pytest.importorskip("torch")
    dec = fi.e4m3_bits_to_f64
    assert dec(0x38) == 1.0 and dec(0x7E) == 448.0 and dec(0xFE) == -448.0
    assert dec(0x08) == 2.0 ** -6 and dec(0x01) == 2.0 ** -9 and dec(0x07) == 7 * 2.0 ** -9
    assert dec(0x00) == 0.0 and np.signbit(dec(0x80)) and dec(0x40) == 2.0
    assert dec(0x3C) == 1.5 and dec(0x77) == 240.0 and dec(0x78) == 256.0
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = dec(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[~np.isnan(mine)], ref[~np.isnan(ref)])


def test_e4m3_encoding_rounds_to_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    codes = np.arange(256, dtype=np.uint8)
    finite = fi.e4m3_bits_to_f64(codes[(codes & 0x7F) != 0x7F])
    pos = np.sort(fi.e4m3_bits_to_f64(codes[:127]))
    x = np.concatenate([rng.standard_normal(20000) * np.exp(rng.uniform(-12, 6, 20000)),
                        finite, (pos[:-1] + pos[1:]) / 2, -(pos[:-1] + pos[1:]) / 2])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fi.f64_to_e4m3_bits(x), ref)
    assert fi.f64_to_e4m3_bits(1.0 + 2.0 ** -4) == 0x38      # tie to the even mantissa 0
    assert fi.f64_to_e4m3_bits(1.0 + 3 * 2.0 ** -4) == 0x3A  # tie to the even mantissa 2
    with pytest.raises(ValueError):
        fi.f64_to_e4m3_bits(465.0)


def test_fp8_generator_codes_dequantise_to_the_draws():
    cfg = dataclasses.replace(fi.CONFIGS[3], N=64, H=2, dtype="e4m3")
    for name in ("q", "k", "v"):
        codes = fi.make_head(cfg, name, 0, 1, seed=3)
        assert codes.dtype == np.uint8 and codes.shape == (64, 128)
        x = fi.make_head(dataclasses.replace(cfg, dtype="f32"), name, 0, 1, seed=3)
        deq = fi.widen(codes, "e4m3") * fi.FP8_DESCALE[name]
        # nearest E4M3 value: relative error at most 2^-4 (normals)
        assert np.all(np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * fi.FP8_DESCALE[name])
        assert np.max(np.abs(fi.widen(codes, "e4m3"))) <= 448
