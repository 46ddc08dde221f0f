"""Parity of the rectangular backward (fa_bwd_rect: Nq query rows against Nk
keys, query row i at position Nk - Nq + i, bottom-right causal) against the
fp64 oracle, through the C ABI.

The GPU backward consumes the GPU forward's (fa_fwd_rect) O and logsumexp, as
a caller would; the oracle computes the exact gradients from q, k, v and dO.
Small shapes (Nq < Nk, Nq > Nk with rows that see no key, a single key,
ragged tiles, shared K/V heads, both d) are compared on every element; the
chunked-prefill workload on whole heads of one K/V group plus dQ on sampled
rows of every head.
"""
import concurrent.futures as cf

import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import check_bf16, sample_rows, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    from exact_attention_41_amd import _lib
    _lib.load()
    return fa


def _run(fa, inp, causal, scale):
    import torch
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.fa_fwd_rect(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd_rect(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(dq), to_np(dk), to_np(dv)


SMALL = [(1, 2, 1, 100, 300, 128), (2, 4, 2, 300, 100, 64), (1, 2, 2, 64, 1000, 128),
         (1, 1, 1, 1, 500, 128), (1, 2, 1, 513, 1025, 64), (1, 3, 3, 700, 333, 128),
         (2, 2, 1, 257, 257, 128), (1, 2, 1, 200, 64, 128), (1, 1, 1, 129, 1, 64)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d", SMALL)
def test_rect_backward_small(fa, B, H, Hkv, Nq, Nk, d, causal):
    say(f"fa_bwd_rect B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} seed=91")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, d, seed=91, with_do=True)
    scale = float(np.float32(1 / np.sqrt(d)))
    dq, dk, dv = _run(fa, inp, causal, scale)
    q64, k64, v64, do64 = inp.as_float64()
    rq, rk, rv = ora.rect_bwd(q64, k64, v64, do64, causal, scale, workers=None)
    check_bf16("dQ", dq, rq)
    check_bf16("dK", dk, rk)
    check_bf16("dV", dv, rv)
    if causal and Nq > Nk:
        assert np.all(dq[:, :, :Nq - Nk] == 0.0), "rows that see no key must get dQ = 0"


def test_rect_backward_matches_square_entry_when_nq_equals_nk(fa):
    """Nq == Nk: fa_bwd_rect and fa_bwd_gqa give identical bits."""
    import torch
    B, H, Hkv, N, d = 1, 4, 2, 300, 128
    say(f"fa_bwd_rect vs fa_bwd_gqa B={B} H={H} Hkv={Hkv} N={N} d={d} seed=92")
    inp = wl.make_decode_inputs(B, H, Hkv, N, N, d, seed=92, with_do=True)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.fa_fwd_gqa(q, k, v, causal=True)
    a = fa.fa_bwd_rect(q, k, v, o, do, lse, causal=True)
    b = fa.fa_bwd_gqa(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_rect_backward_prefill_workload(fa):
    """The chunked-prefill shape (4096 new queries after 12288 cached keys,
    32 query heads on 8 K/V heads): dK, dV of one K/V head and dQ of its four
    query heads element by element, plus dQ on sampled rows of every head."""
    w = wl.RECT_WORKLOADS["bf16_prefill_b1h32kv8q4096k16384d128_causal"]
    G = w.H // w.Hkv
    say(f"rect bwd workload {w.name}: B={w.B} H={w.H} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d}")
    inp = wl.make_decode_inputs(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed, with_do=True)
    dq, dk, dv = _run(fa, inp, w.causal, w.scale)
    q64, k64, v64, do64 = inp.as_float64()
    kvh = 5
    heads = [(0, kvh * G + g) for g in range(G)]
    rq, rk, rv = ora.rect_bwd(q64, k64, v64, do64, w.causal, w.scale, heads=heads, workers=None)
    check_bf16("dQ (one K/V group)", dq[0, kvh * G:(kvh + 1) * G], rq)
    check_bf16("dK (one K/V head)", dk[0, kvh], rk.sum(axis=0))
    check_bf16("dV (one K/V head)", dv[0, kvh], rv.sum(axis=0))
    rows = sample_rows(w.Nq, 32, seed=w.seed)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        return ora.head_dq_rows(q64[b, h], k64[b, h // G], v64[b, h // G], do64[b, h], w.causal,
                                w.scale, rows, pos0=w.Nk - w.Nq)

    with cf.ThreadPoolExecutor(8) as ex:
        ref = np.stack(list(ex.map(one, pairs)))
    check_bf16("dQ (sampled rows, all heads)", dq.reshape(w.B * w.H, w.Nq, w.d)[:, rows], ref)
