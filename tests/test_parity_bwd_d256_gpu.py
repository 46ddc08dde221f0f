"""Parity of the backward at head size 256 (fa_bwd, fa_bwd_gqa, fa_bwd_rect
with d = 256) against the fp64 oracle, through the C ABI.

The GPU backward consumes the GPU forward's O and logsumexp. Small shapes
(several query blocks and key tiles, ragged tails, Nq != Nk with bottom-right
causal alignment and rows that see no key, shared K/V heads) are compared on
every element; the head-size-256 benchmark workload on two whole heads plus dQ
on sampled rows of every head. Both ways of forming D are tested: from O and
the forward's rounding residual ("o_res"), and in the dQ pass ("exact").
"""
import concurrent.futures as cf

import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import check_bf16, sample_rows, say, to_np

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


MODES = ["o_res", "exact"]


def _fwd_bwd(fa, inp, causal, scale, mode):
    import torch
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o_res = torch.empty_like(q) if mode == "o_res" else None
    o, lse = fa.fa_fwd_rect(q, k, v, causal=causal, scale=scale, o_res=o_res)
    dq, dk, dv = fa.fa_bwd_rect(q, k, v, o, do, lse, causal=causal, scale=scale, o_res=o_res)
    torch.cuda.synchronize()
    return to_np(dq), to_np(dk), to_np(dv)


SMALL = [(1, 2, 2, 300, 300), (2, 2, 1, 129, 129), (1, 4, 2, 200, 517), (1, 2, 1, 300, 100),
         (1, 1, 1, 1, 1), (1, 1, 1, 64, 64), (1, 2, 2, 520, 520)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk", SMALL)
def test_d256_backward_small(fa, B, H, Hkv, Nq, Nk, causal, mode):
    say(f"d=256 backward B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} D from {mode} "
        f"seed=93")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, D, seed=93, with_do=True)
    scale = float(np.float32(1 / np.sqrt(D)))
    dq, dk, dv = _fwd_bwd(fa, inp, causal, scale, mode)
    q64, k64, v64, do64 = inp.as_float64()
    rq, rk, rv = ora.rect_bwd(q64, k64, v64, do64, causal, scale, workers=None)
    check_bf16("dQ", dq, rq)
    check_bf16("dK", dk, rk)
    check_bf16("dV", dv, rv)


# Grids large enough for the passes with 16-row steps (at least 256
# workgroups of 128 keys for dK/dV, of 128 query rows for dQ when D comes
# from the residual): ragged key blocks and query tiles, shared K/V heads,
# Nq < Nk and Nq > Nk with bottom-right causal alignment.
LARGE_GRID = [(1, 128, 128, 300, 300), (1, 256, 128, 200, 517), (2, 64, 64, 333, 190)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk", LARGE_GRID)
def test_d256_backward_large_grid(fa, B, H, Hkv, Nq, Nk, causal, mode):
    say(f"d=256 backward (16-row-step passes) B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} "
        f"causal={causal} D from {mode} seed=95")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, D, seed=95, with_do=True)
    scale = float(np.float32(1 / np.sqrt(D)))
    dq, dk, dv = _fwd_bwd(fa, inp, causal, scale, mode)
    q64, k64, v64, do64 = inp.as_float64()
    rq, rk, rv = ora.rect_bwd(q64, k64, v64, do64, causal, scale, workers=None)
    check_bf16("dQ", dq, rq)
    check_bf16("dK", dk, rk)
    check_bf16("dV", dv, rv)


def test_d256_backward_square_entries_agree(fa):
    """fa_bwd and fa_bwd_rect (Nq = Nk) give identical bits at d = 256, and
    repeated calls give identical bits."""
    import torch
    B, H, N = 1, 2, 333
    say(f"d=256 fa_bwd vs fa_bwd_rect B={B} H={H} N={N} seed=94")
    inp = wl.make_inputs(B, H, N, D, "bf16", seed=94, with_do=True)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    a = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    b = fa.fa_bwd_rect(q, k, v, o, do, lse, causal=True)
    c = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name", list(wl.WIDE_WORKLOADS))
def test_d256_backward_workload(fa, name, mode):
    """B=4 H=8 N=4096 d=256 (both masks): two whole heads element by element,
    plus dQ on sampled rows of every head."""
    w = wl.WIDE_WORKLOADS[name]
    say(f"d=256 backward workload {w.name}: B={w.B} H={w.H} N={w.N} causal={w.causal} "
        f"D from {mode}")
    inp = wl.make_inputs(w.B, w.H, w.N, w.d, "bf16", w.seed, with_do=True)
    dq, dk, dv = _fwd_bwd(fa, inp, w.causal, w.scale, mode)
    gq, gk, gv = (x.reshape(w.B * w.H, w.N, w.d) for x in (dq, dk, dv))
    q64, k64, v64, do64 = inp.as_float64()
    heads = [(0, 3), (3, 6)]
    rq, rk, rv = ora.attention_bwd(q64, k64, v64, do64, w.causal, w.scale, heads=heads,
                                   workers=None)
    idx = [b * w.H + h for b, h in heads]
    check_bf16("dQ (2 heads)", gq[idx], rq)
    check_bf16("dK (2 heads)", gk[idx], rk)
    check_bf16("dV (2 heads)", gv[idx], rv)
    rows = sample_rows(w.N, 24, seed=w.seed)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        return ora.head_dq_rows(q64[b, h], k64[b, h], v64[b, h], do64[b, h], w.causal,
                                w.scale, rows)

    with cf.ThreadPoolExecutor(8) as ex:
        ref = np.stack(list(ex.map(one, pairs)))
    check_bf16("dQ (sampled rows, all heads)", gq[:, rows], ref)
