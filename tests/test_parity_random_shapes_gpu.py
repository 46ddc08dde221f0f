"""Seeded random shapes through the bf16 forward and backward (fa_fwd_rect,
fa_bwd_rect), every element against the fp64 oracle: batch, heads, shared
K/V heads, Nq, Nk (including Nq > Nk and single rows), head size and mask
drawn from one fixed generator, so the set is the same on every run."""
import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import LSE_ATOL, check_abs, check_bf16, say, to_np

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=2024):
    r = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        B = int(r.integers(1, 3))
        Hkv = int(r.integers(1, 4))
        H = Hkv * int(r.choice([1, 2, 4]))
        d = int(r.choice([64, 128, 256]))
        Nq = int(r.choice([1, 2, 63, 64, 65]) if i % 4 == 0 else r.integers(1, 400))
        Nk = int(r.choice([1, 31, 64, 129]) if i % 5 == 0 else r.integers(1, 600))
        causal = bool(r.integers(0, 2))
        out.append((i, B, H, Hkv, Nq, Nk, d, causal))
    return out


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    from exact_attention_41_amd import _lib
    _lib.load()
    return fa


@pytest.mark.parametrize("i,B,H,Hkv,Nq,Nk,d,causal", _cases())
def test_random_shape_forward_and_backward(fa, i, B, H, Hkv, Nq, Nk, d, causal):
    import torch
    say(f"random case {i}: B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} "
        f"seed={300 + i}")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, d, seed=300 + i, with_do=True)
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.fa_fwd_rect(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd_rect(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = inp.as_float64()
    ro, rl = ora.rect_fwd(q64, k64, v64, causal, scale, workers=None)
    rq, rk, rv = ora.rect_bwd(q64, k64, v64, do64, causal, scale, workers=None)
    check_bf16("O", to_np(o), ro)
    check_abs("lse", to_np(lse), rl, LSE_ATOL)
    check_bf16("dQ", to_np(dq), rq)
    check_bf16("dK", to_np(dk), rk)
    check_bf16("dV", to_np(dv), rv)


def test_backward_phases_equal_fa_bwd_at_d256(fa):
    """At d = 256 too, fa_bwd is exactly its three phases."""
    import torch
    B, H, N, d = 1, 2, 200, 256
    say(f"fa_bwd phases d={d} B={B} H={H} N={N} causal=True seed=95")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=95, with_do=True)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    dq1, dk1, dv1 = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=q.device)
    dq2, dk2, dv2 = (torch.empty_like(q) for _ in range(3))
    fa.fa_bwd_preprocess(q, k, v, o, do, ws)
    fa.fa_bwd_dq(q, k, v, do, lse, ws, dq2, causal=True)
    fa.fa_bwd_dkdv(q, k, v, do, ws, dk2, dv2, causal=True)
    torch.cuda.synchronize()
    for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2)):
        assert torch.equal(a, b)
