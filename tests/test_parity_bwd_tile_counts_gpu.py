"""Backward parity at whole-tile sizes: every number of 64-row tiles from one to
five, through fa_bwd_gqa (shared K/V heads, groups of one and two) against the
fp64 oracle, at head sizes 64, 128 and 256.

The dQ pass cycles its key tiles through three LDS buffers and the dK/dV pass
cycles row-major tiles by step, images by query tile and statistics through
three buffers, walking the query tiles of every head of a group in turn. One to
five tiles (times one or two heads per group, times one or two column steps at
d = 256) take every buffer through its first use, its wrap-around and the
change of group member, at sizes small enough to compare every element.
"""
import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import check_bf16, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    from exact_attention_41_amd import _lib
    _lib.load()
    return fa


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("tiles", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_whole_tiles(fa, d, tiles, G, causal):
    import torch
    B, Hkv, N = 1, 2, 64 * tiles
    H = G * Hkv
    say(f"fa_bwd_gqa B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} seed=41")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=41, with_do=True, Hkv=Hkv)
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.fa_fwd_gqa(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd_gqa(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = inp.as_float64()
    rq, rk, rv = ora.attention_bwd(q64, k64, v64, do64, causal, scale, workers=None)
    check_bf16("dQ", to_np(dq), rq)
    check_bf16("dK", to_np(dk), rk)
    check_bf16("dV", to_np(dv), rv)
