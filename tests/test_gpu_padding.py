"""Key and value rows at or past a sequence's key length are never read:
filling them with NaN changes no output bit (forward, backward, FP8
forward), and their dK, dV rows are zero."""

import numpy as np
import pytest

import fa_inputs as fi
from tests.gpu_helpers import custom, lib, log_case, to_device, torch_cuda

pytestmark = pytest.mark.gpu

LENGTHS = [0, 5, 130, 253]   # N = 256: empty, short, ragged, almost full


def poisoned(t, lengths, fill):
    out = t.copy()
    for b, n in enumerate(lengths):
        out[b, :, n:] = fill
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_padding_changes_nothing(dtype, causal):
    torch = torch_cuda()
    fa = lib()
    log_case(test="nan-padding", dtype=dtype, causal=causal)
    cfg = custom(5, B=len(LENGTHS), H=2, N=256, d=128, dtype=dtype)
    t = {n: fi.make_tensor(cfg, n, 9) for n in ("q", "k", "v", "do")}
    nan = {"bf16": 0x7FC0, "f16": 0x7E00, "f32": np.float32(np.nan)}[dtype]
    lens = torch.from_numpy(np.array(LENGTHS, np.int32)).cuda()
    results = []
    for fill in (0, nan):
        dev = {n: to_device(torch, t[n], dtype) for n in t}
        for n in ("k", "v"):
            dev[n] = to_device(torch, poisoned(t[n], LENGTHS, fill), dtype)
        o, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal=causal, seqlens_k=lens)
        g = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal,
                        seqlens_k=lens)
        torch.cuda.synchronize()
        results.append((o, lse) + tuple(g))
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), results[0], results[1]):
        assert torch.equal(a, b), name
    for b, n in enumerate(LENGTHS):
        assert torch.count_nonzero(results[1][3][b, :, n:]).item() == 0
        assert torch.count_nonzero(results[1][4][b, :, n:]).item() == 0


def test_fp8_nan_padding_changes_nothing():
    torch = torch_cuda()
    fa = lib()
    log_case(test="nan-padding-fp8")
    cfg = custom(3, B=len(LENGTHS), H=2, N=256, dtype="e4m3")
    codes = {n: fi.make_tensor(cfg, n, 4) for n in "qkv"}
    lens = torch.from_numpy(np.array(LENGTHS, np.int32)).cuda()
    outs = []
    for fill in (0, 0x7F):   # 0x7F: the E4M3 NaN
        dev = {n: torch.from_numpy(codes[n] if n == "q" else poisoned(codes[n], LENGTHS, fill))
               .cuda() for n in "qkv"}
        outs.append(fa.forward_fp8(dev["q"], dev["k"], dev["v"], fi.FP8_DESCALE["q"],
                                   fi.FP8_DESCALE["k"], fi.FP8_DESCALE["v"], causal=True,
                                   seqlens_k=lens))
        torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
