"""Parity of head size 256 (the bf16 forward entry points and decoding) against
the fp64 oracle, through the C ABI.

Small shapes (several 128-row query blocks and 64-key tiles, ragged tails,
Nq != Nk with bottom-right causal alignment, shared K/V heads) are compared on
every element. One case gives later key tiles scores far above the first
tile's, so that rows which already hold a sum must move their reference
maximum (the output accumulator is rescaled). The benchmark workloads are
compared on sampled rows of every head, decoding on every row.
"""
import concurrent.futures as cf

import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import LSE_ATOL, check_abs, check_bf16, sample_rows, say, to_np

pytestmark = pytest.mark.gpu

D = 256


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    from exact_attention_41_amd import _lib
    _lib.load()
    return fa


def _forward(fa, inp, causal, scale, Nq, Nk, H, Hkv):
    import torch
    q, k, v = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    if Nq == Nk and H == Hkv:
        o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    else:
        o, lse = fa.fa_fwd_rect(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


SMALL = [(1, 2, 2, 300, 300), (2, 2, 1, 129, 129), (1, 4, 2, 200, 517), (1, 2, 1, 300, 100),
         (1, 1, 1, 1, 1), (1, 1, 1, 64, 64), (1, 3, 1, 257, 1000), (1, 2, 2, 520, 520)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk", SMALL)
def test_d256_forward_small(fa, B, H, Hkv, Nq, Nk, causal):
    say(f"d=256 forward B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} seed=91")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, D, seed=91)
    scale = float(np.float32(1 / np.sqrt(D)))
    o, lse = _forward(fa, inp, causal, scale, Nq, Nk, H, Hkv)
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.rect_fwd(q64, k64, v64, causal, scale, workers=None)
    check_bf16("O", o, ro)
    check_abs("lse", lse, rl, LSE_ATOL)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_d256_forward_rescales_rows_holding_a_sum(fa, causal):
    """Keys 128..255 multiplied by 2^5 and keys from 256 on by 2^8 (exact in
    bf16): their scores exceed the first tiles' maxima by far more than the
    reference-maximum threshold, after the rows have accumulated a sum."""
    B, H, N = 1, 2, 640
    say(f"d=256 forward, growing key scale B={B} H={H} N={N} causal={causal} seed=92")
    inp = wl.make_decode_inputs(B, H, H, N, N, D, seed=92)
    k = inp.k.copy()
    k[:, :, 128:256] *= 32.0
    k[:, :, 256:] *= 256.0
    inp = wl.Inputs(inp.q, k, inp.v, None, "bf16")
    scale = float(np.float32(1 / np.sqrt(D)))
    o, lse = _forward(fa, inp, causal, scale, N, N, H, H)
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.rect_fwd(q64, k64, v64, causal, scale, workers=None)
    check_bf16("O", o, ro)
    check_abs("lse", lse, rl, LSE_ATOL)


@pytest.mark.parametrize("name", list(wl.WIDE_WORKLOADS))
def test_d256_forward_workload(fa, name):
    """B=4 H=8 N=4096 d=256 in the benchmark's launch: sampled rows of every
    head."""
    w = wl.WIDE_WORKLOADS[name]
    say(f"d=256 workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    inp = wl.workload_inputs(w)
    o, lse = _forward(fa, inp, w.causal, w.scale, w.N, w.N, w.H, w.H)
    q64, k64, v64, _ = inp.as_float64()
    rows = sample_rows(w.N, 40, seed=w.seed)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    ro, rl = ora.attention_fwd(q64, k64, v64, w.causal, w.scale, heads=pairs, rows=rows,
                               workers=None)
    check_bf16("O (sampled rows, all heads)", o.reshape(w.B * w.H, w.N, w.d)[:, rows], ro)
    check_abs("lse (sampled rows, all heads)", lse.reshape(w.B * w.H, w.N)[:, rows], rl,
              LSE_ATOL)


def _decode(fa, inp, causal, scale):
    import torch
    q, k, v = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o, lse = fa.fa_decode(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


DEC_SMALL = [(1, 4, 1, 1, 1000), (2, 8, 2, 4, 777), (1, 32, 1, 1, 5000), (1, 2, 2, 3, 3)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk", DEC_SMALL)
def test_d256_decode_small(fa, B, H, Hkv, Nq, Nk, causal):
    say(f"d=256 fa_decode B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} seed=93")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, D, seed=93)
    scale = float(np.float32(1 / np.sqrt(D)))
    o, lse = _decode(fa, inp, causal, scale)
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.decode_fwd(q64, k64, v64, causal, scale, workers=None)
    check_bf16("O", o, ro)
    check_abs("lse", lse, rl, LSE_ATOL)


def test_d256_decode_workload(fa):
    w = wl.DECODE_WORKLOADS["bf16_decode_b8h16kv4q1k32768d256"]
    say(f"decode workload {w.name}: B={w.B} H={w.H} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d}")
    inp = wl.make_decode_inputs(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed)
    o, lse = _decode(fa, inp, w.causal, w.scale)
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.decode_fwd(q64, k64, v64, w.causal, w.scale, workers=None)
    check_bf16("O (every row)", o, ro)
    check_abs("lse (every row)", lse, rl, LSE_ATOL)
