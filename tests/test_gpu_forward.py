"""Forward parity on the GPU: fa_forward through the C ABI against the fp64
oracle on the same seeded inputs.

Tolerances: O max-abs <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 and <= 5e-3
for f16 (its unit roundoff is 1/8 of bf16's; the bound keeps a margin for the
fp32 accumulation order); LSE <= 1e-5 abs for fp32, <= ln(1 + 2^-8) + 1e-4
+ 1e-5 |LSE| for bf16 and <= 1e-3 + 1e-5 |LSE| for f16 (the running sum adds
the weights rounded to the MFMA operand format); empty rows must give O == 0
and LSE == -inf exactly.
"""

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_helpers import (LSE_TOL, check_lse, custom, device_inputs, from_device, lib,
                               log_case, max_abs, parallel_map, torch_cuda)

pytestmark = pytest.mark.gpu

O_TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 5e-3}


def run_forward(torch, cfg, inputs, stream=None):
    fa = lib()
    dev = device_inputs(torch, cfg, inputs)
    if stream is None:
        o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=cfg.causal,
                            seqlens_k=dev["lengths"])
    else:
        with torch.cuda.stream(stream):
            o, lse = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale,
                                causal=cfg.causal, seqlens_k=dev["lengths"])
    torch.cuda.synchronize()
    return from_device(o, cfg.dtype), lse.cpu().numpy().astype(np.float64)


def widen_all(cfg, inputs):
    return [fi.widen(inputs[n], cfg.dtype) for n in ("q", "k", "v")]


def assert_forward_close(cfg, o, lse, ref_o, ref_lse):
    assert not np.any(np.isnan(o))
    err = max_abs(o, ref_o)
    assert err <= O_TOL[cfg.dtype], f"O max abs error {err:.3e}"
    check_lse(lse, ref_lse, *LSE_TOL[cfg.dtype])
    empty = np.isneginf(ref_lse)
    assert np.all(o[empty] == 0.0)
    return err


def test_config1_fp32_full_against_both_routes():
    torch = torch_cuda()
    cfg = fi.CONFIGS[1]
    log_case(test="config1", shape=cfg.shape, dtype=cfg.dtype)
    inputs = fi.make_inputs(cfg)
    o, lse = run_forward(torch, cfg, inputs)
    q, k, v = widen_all(cfg, inputs)
    ra_o, ra_l = oracle.attention_materialised(q, k, v, cfg.scale)
    rb_o, rb_l = oracle.attention_online(q, k, v, cfg.scale, tile=64)
    assert_forward_close(cfg, o, lse, ra_o, ra_l)
    assert_forward_close(cfg, o, lse, rb_o, rb_l)


SMALL_N = [1, 2, 63, 65, 127, 129, 256, 300, 513]


@pytest.mark.parametrize("d", [64, 96, 128, 192, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_small_shapes_all_rows(d, causal, dtype):
    """Ragged N across several tiles, every length edge case, every row."""
    torch = torch_cuda()
    for N in SMALL_N:
        for lens_kind in ("none", "edges", "random"):
            if lens_kind == "none":
                lengths = None
            elif lens_kind == "edges":
                lengths = np.array([0, 1, N, max(N - 1, 0)], np.int32)
            else:
                lengths = np.random.default_rng(N).integers(0, N + 1, 4).astype(np.int32)
            B = 4 if lengths is not None else 2
            cfg = custom(2, B=B, H=3, N=N, d=d, dtype=dtype, causal=causal)
            log_case(test="small", N=N, d=d, causal=causal, dtype=dtype, lengths=lens_kind)
            inputs = fi.make_inputs(cfg, seed=N)
            inputs["lengths"] = lengths
            o, lse = run_forward(torch, cfg, inputs)
            q, k, v = widen_all(cfg, inputs)
            ref_o, ref_l = oracle.attention_materialised(q, k, v, cfg.scale, causal, lengths)
            assert_forward_close(cfg, o, lse, ref_o, ref_l)


@pytest.mark.parametrize("causal", [False, True])
def test_f32_d64_small_and_large_grids(causal):
    """fp32 at d = 64 takes two paths by grid size: below the CU count each
    64-row block's keys are split over four waves whose partial states are
    merged at the end; above it one wave per 32-row block walks every key.
    A 288-work-group batch (ragged lengths, an empty sequence) runs the
    second path; each of two of its heads alone runs the first; all match
    the oracle on every row."""
    torch = torch_cuda()
    cfg = custom(2, B=2, H=16, N=520, d=64, dtype="f32", causal=causal)
    log_case(test="f32_d64_grids", shape=cfg.shape, causal=causal)
    inputs = fi.make_inputs(cfg, seed=11)
    inputs["lengths"] = np.array([0, 389], np.int32)
    o, lse = run_forward(torch, cfg, inputs)
    q, k, v = widen_all(cfg, inputs)
    ref_o, ref_l = oracle.attention_materialised(q, k, v, cfg.scale, causal, inputs["lengths"])
    assert_forward_close(cfg, o, lse, ref_o, ref_l)
    for b, h in ((1, 0), (1, 15)):
        one = custom(2, B=1, H=1, N=520, d=64, dtype="f32", causal=causal)
        sub = {n: np.ascontiguousarray(inputs[n][b:b + 1, h:h + 1]) for n in ("q", "k", "v")}
        sub["lengths"] = inputs["lengths"][b:b + 1].copy()
        o1, l1 = run_forward(torch, one, sub)
        assert_forward_close(one, o1, l1, ref_o[b:b + 1, h:h + 1], ref_l[b:b + 1, h:h + 1])


def test_lengths_clamped_to_range():
    torch = torch_cuda()
    cfg = custom(2, B=3, H=2, N=130, causal=True)
    inputs = fi.make_inputs(cfg, seed=5)
    inputs["lengths"] = np.array([-7, 500, 64], np.int32)
    o, lse = run_forward(torch, cfg, inputs)
    q, k, v = widen_all(cfg, inputs)
    ref_o, ref_l = oracle.attention_materialised(q, k, v, cfg.scale, True,
                                                 np.array([0, 130, 64]))
    assert_forward_close(cfg, o, lse, ref_o, ref_l)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_config2_full(dtype):
    torch = torch_cuda()
    cfg = custom(2, dtype=dtype)
    log_case(test="config2", shape=cfg.shape, dtype=dtype)
    inputs = fi.make_inputs(cfg)
    o, lse = run_forward(torch, cfg, inputs)
    q, k, v = widen_all(cfg, inputs)
    ref_o, ref_l = oracle.attention_materialised(q, k, v, cfg.scale, False)
    err = assert_forward_close(cfg, o, lse, ref_o, ref_l)
    print(f"config2 {dtype} O max abs err {err:.3e}", flush=True)


def _sampled_rows(rng, N, extra=()):
    rows = set(rng.choice(N, size=min(N, 64), replace=False).tolist())
    for t in (64, 128, 256):
        for base in range(0, N, 1024):
            for r in (base + t - 1, base + t):
                if 0 <= r < N:
                    rows.add(r)
    rows.update(r for r in extra if 0 <= r < N)
    rows.update({0, N - 1})
    return np.array(sorted(rows))


def oracle_heads_all_rows(cfg, inputs, heads, lengths=None, chunk=256):
    """Route A on every row of the given (b, h) heads, the rows of all heads
    cut into chunks that run in parallel on the host's cores.  Returns
    {(b, h): (o, lse)}."""
    wide = {(b, h): [fi.widen(inputs[n][b, h], cfg.dtype) for n in ("q", "k", "v")]
            for (b, h) in heads}
    N = cfg.N
    jobs = [(b, h, r0) for (b, h) in heads for r0 in range(0, N, chunk)]

    def run(job):
        b, h, r0 = job
        q, k, v = wide[(b, h)]
        rows = np.arange(r0, min(N, r0 + chunk))
        length = None if lengths is None else int(lengths[b])
        return oracle.attention_rows(q, k, v, rows, cfg.scale, cfg.causal, length)

    res = parallel_map(run, jobs)
    out = {}
    for (b, h) in heads:
        parts = [r for (jb, jh, _), r in zip(jobs, res) if (jb, jh) == (b, h)]
        out[(b, h)] = (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    return out


def test_config3_every_head_every_row():
    """The causal N=8192 forward: all 32 heads, all 8192 rows each, against
    route A (row-blocked only to spread it over the host's cores)."""
    torch = torch_cuda()
    cfg = fi.CONFIGS[3]
    log_case(test="config3", shape=cfg.shape)
    inputs = fi.make_inputs(cfg)
    o, lse = run_forward(torch, cfg, inputs)
    assert not np.any(np.isnan(o)) and not np.any(np.isnan(lse))
    heads = [(0, h) for h in range(cfg.H)]
    ref = oracle_heads_all_rows(cfg, inputs, heads)
    worst = 0.0
    worst_lse = 0.0
    for (b, h) in heads:
        ref_o, ref_l = ref[(b, h)]
        worst = max(worst, assert_forward_close(cfg, o[b, h], lse[b, h], ref_o, ref_l))
        worst_lse = max(worst_lse, check_lse(lse[b, h], ref_l, *LSE_TOL[cfg.dtype]))
    print(f"config3 all 32 heads x 8192 rows: O max abs err {worst:.3e}, "
          f"LSE max abs err {worst_lse:.3e}", flush=True)


def test_config4_focus_heads_every_row_and_every_head_sampled():
    """Key lengths with x30 queries at padded N=32768: the empty sequence
    exactly (O = 0, LSE = -inf on every row of every head); every row of the
    heads h in {0, 31} of the shortest non-empty and the longest sequence;
    and in every (b, h) 64 random rows, the rows L_b - 1 and L_b and the rows
    on both sides of each 64/128/256-row tile edge every 1024 rows."""
    torch = torch_cuda()
    fa = lib()
    cfg = fi.CONFIGS[4]
    log_case(test="config4", shape=cfg.shape)
    inputs = fi.make_inputs(cfg)
    L = inputs["lengths"]
    dev = device_inputs(torch, cfg, inputs)
    o_dev, lse_dev = fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=True,
                                seqlens_k=dev["lengths"])
    torch.cuda.synchronize()
    del dev
    lse = lse_dev.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(lse))
    # the length-0 sequence: every row empty, O exactly zero
    b_empty = int(np.argmin(L))
    assert L[b_empty] == 0
    assert np.all(np.isneginf(lse[b_empty]))
    assert torch.count_nonzero(o_dev[b_empty].view(torch.int16)).item() == 0
    nonempty = [b for b in range(cfg.B) if L[b] > 0]
    assert not np.any(np.isneginf(lse[nonempty]))
    assert not torch.isnan(o_dev).any().item()
    b_small = int(np.argmin(np.where(L > 0, L, cfg.N + 1)))
    b_large = int(np.argmax(L))
    focus = [(b, h) for b in (b_small, b_large) for h in (0, 31)]
    worst = 0.0
    ref = oracle_heads_all_rows(cfg, inputs, focus, lengths=L)
    for (b, h) in focus:
        ref_o, ref_l = ref[(b, h)]
        got = from_device(o_dev[b, h], "bf16")
        worst = max(worst, assert_forward_close(cfg, got, lse[b, h], ref_o, ref_l))
    print(f"config4 focus heads {focus} all rows: O max abs err {worst:.3e}", flush=True)
    rng = np.random.default_rng(4)
    jobs = []
    for b in nonempty:
        Lb = int(L[b])
        for h in range(cfg.H):
            jobs.append((b, h, _sampled_rows(rng, cfg.N, [Lb - 1, Lb])))

    def run(job):
        b, h, rows = job
        q, k, v = (fi.widen(inputs[n][b, h], "bf16") for n in ("q", "k", "v"))
        return oracle.attention_rows(q, k, v, rows, cfg.scale, True, int(L[b]))

    refs = parallel_map(run, jobs)
    for (b, h, rows), (ref_o, ref_l) in zip(jobs, refs):
        got = from_device(o_dev[b, h][torch.from_numpy(rows).cuda()], "bf16")
        worst = max(worst, assert_forward_close(cfg, got, lse[b, h, rows], ref_o, ref_l))
    assert np.max(np.abs(lse[nonempty])) > 60.0      # the x30 scores really are large
    print(f"config4 O max abs err {worst:.3e} ({len(jobs)} sampled heads)", flush=True)


def test_forward_is_deterministic_and_stream_aware():
    torch = torch_cuda()
    cfg = custom(3, B=1, H=4, N=1000)
    inputs = fi.make_inputs(cfg, seed=9)
    o1, l1 = run_forward(torch, cfg, inputs)
    s = torch.cuda.Stream()
    o2, l2 = run_forward(torch, cfg, inputs, stream=s)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_forward_writes_nothing_outside_outputs():
    torch = torch_cuda()
    fa = lib()
    cfg = custom(3, B=2, H=2, N=77)
    inputs = fi.make_inputs(cfg, seed=2)
    dev = device_inputs(torch, cfg, inputs)
    n = cfg.B * cfg.H * cfg.N * cfg.d
    pad = 4096
    o_buf = torch.full((n + pad,), -7.0, dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((cfg.B * cfg.H * cfg.N + pad,), -7.0, dtype=torch.float32, device="cuda")
    o = o_buf[:n].view(cfg.shape)
    lse = l_buf[:cfg.B * cfg.H * cfg.N].view(cfg.B, cfg.H, cfg.N)
    fa.forward(dev["q"], dev["k"], dev["v"], scale=cfg.scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o_buf[n:] == -7.0).item()
    assert torch.all(l_buf[cfg.B * cfg.H * cfg.N:] == -7.0).item()
    ref_o, ref_l = oracle.attention_materialised(*(fi.widen(inputs[x], "bf16") for x in "qkv"),
                                                 cfg.scale, True)
    assert_forward_close(cfg, from_device(o, "bf16"), lse.cpu().numpy().astype(np.float64),
                         ref_o, ref_l)


def test_peak_memory_grows_linearly():
    """Only the I/O tensors are allocated: doubling N doubles peak memory."""
    torch = torch_cuda()
    fa = lib()
    peaks = []
    for N in (8192, 16384):
        torch.cuda.empty_cache()
        q = torch.randn(1, 8, N, 128, device="cuda").to(torch.bfloat16)
        k = torch.randn_like(q)
        v = torch.randn_like(q)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        fa.forward(q, k, v, causal=True)
        torch.cuda.synchronize()
        peaks.append(torch.cuda.max_memory_allocated() - base)
        del q, k, v
    # O (N*d*2 B per head) plus LSE (4 B per row): exactly linear in N
    assert peaks[1] <= 2.05 * peaks[0]
    assert peaks[0] <= 8 * 8192 * (128 * 2 + 4) * 1.1
