"""Backward parity: fa_bwd (through the C ABI) against the fp64 oracle.

The GPU backward consumes the GPU forward's O and logsumexp, as a caller
would; the oracle computes the exact gradients of sum(O * dO) from q, k, v
and dO alone. One isolation case feeds the GPU backward the oracle's own O
(rounded to bf16) and logsumexp (rounded to fp32) instead.

Both ways of forming D_i = dO_i . O_i are tested: "o_res" (the forward keeps
O's rounding residual and the preprocess forms D from O plus residual; the
dQ pass takes D from the workspace) and "exact" (no residual: the dQ pass
forms D from P and dP itself).
"""
import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import check_bf16, oracle_workers, say, single_threaded_blas, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    from exact_attention_41_amd import _lib
    _lib.load()
    return fa


MODES = ["o_res", "exact"]


def _gpu_fwd_bwd(fa, inp, causal, scale, mode):
    import torch
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o_res = torch.empty_like(q) if mode == "o_res" else None
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale, o_res=o_res)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale, o_res=o_res)
    torch.cuda.synchronize()
    return dq, dk, dv


SMALL = [(1, 1, 1, 64), (1, 1, 40, 128), (2, 2, 64, 64), (1, 2, 129, 128), (2, 1, 300, 64),
         (1, 2, 300, 128), (1, 1, 700, 128)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,N,d", SMALL)
def test_bf16_backward_small(fa, B, H, N, d, causal, mode):
    say(f"fa_bwd bf16 B={B} H={H} N={N} d={d} causal={causal} D from {mode} seed=21")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=21, with_do=True)
    scale = float(np.float32(1 / np.sqrt(d)))
    dq, dk, dv = _gpu_fwd_bwd(fa, inp, causal, scale, mode)
    q64, k64, v64, do64 = inp.as_float64()
    rq, rk, rv = ora.attention_bwd(q64, k64, v64, do64, causal, scale, workers=None)
    check_bf16("dQ", to_np(dq), rq)
    check_bf16("dK", to_np(dk), rk)
    check_bf16("dV", to_np(dv), rv)


def test_bf16_backward_with_oracle_forward_outputs(fa):
    """Isolation: the backward fed the oracle's O (bf16) and lse (fp32)."""
    import torch
    B, H, N, d, causal = 1, 2, 200, 128, True
    say(f"fa_bwd isolation B={B} H={H} N={N} d={d} causal={causal} seed=22")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=22, with_do=True)
    scale = float(np.float32(1 / np.sqrt(d)))
    q64, k64, v64, do64 = inp.as_float64()
    ro, rl = ora.attention_fwd(q64, k64, v64, causal, scale)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o = wl.to_device(wl.bf16_round(ro.astype(np.float32)), "bf16")
    lse = torch.from_numpy(rl.astype(np.float32)).cuda()
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = ora.attention_bwd(q64, k64, v64, do64, causal, scale)
    check_bf16("dQ", to_np(dq), rq)
    check_bf16("dK", to_np(dk), rk)
    check_bf16("dV", to_np(dv), rv)


def test_bf16_backward_workload(fa):
    """Causal fwd+bwd, B=4 H=16 N=4096 d=128: every element of dQ, dK and dV
    of every head, with D from O and its residual (the training step the
    benchmark times) and with D formed in the dQ pass."""
    w = wl.WORKLOADS["bf16_b4h16n4096d128_causal_bwd"]
    inp = wl.workload_inputs(w)
    q64, k64, v64, do64 = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v, inp.do))
    say(f"  oracle on {oracle_workers()} threads")
    with single_threaded_blas():
        rq, rk, rv = ora.attention_bwd(q64, k64, v64, do64, w.causal, w.scale,
                                       workers=oracle_workers())
    for mode in MODES:
        say(f"fa_bwd workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} seed={w.seed} "
            f"D from {mode}")
        dq, dk, dv = _gpu_fwd_bwd(fa, inp, w.causal, w.scale, mode)
        check_bf16(f"dQ {w.name} ({mode})", to_np(dq), rq)
        check_bf16(f"dK {w.name} ({mode})", to_np(dk), rk)
        check_bf16(f"dV {w.name} ({mode})", to_np(dv), rv)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("v_mean", [8.0, 32.0])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bf16_backward_sharp_scores_large_value_mean(fa, causal, v_mean, mode):
    """Stress inputs outside the specified workloads: q, k x3 (sharp rows) and
    values with a large mean, so |dP| is far larger than |dP - D| (the dQ pass
    subtracts a centre before rounding). Every element of dQ, dK, dV, under
    the "rounded" bf16 rule."""
    B, H, N, d = 1, 4, 1024, 128
    say(f"fa_bwd stress B={B} H={H} N={N} d={d} causal={causal} qk x3 v_mean={v_mean} "
        f"D from {mode} seed=24")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=24, qk_mult=3.0, with_do=True, v_mean=v_mean)
    scale = float(np.float32(1 / np.sqrt(d)))
    dq, dk, dv = _gpu_fwd_bwd(fa, inp, causal, scale, mode)
    q64, k64, v64, do64 = inp.as_float64()
    rq, rk, rv = ora.attention_bwd(q64, k64, v64, do64, causal, scale, workers=None)
    check_bf16("dQ", to_np(dq), rq, rule="rounded")
    check_bf16("dK", to_np(dk), rk, rule="rounded")
    check_bf16("dV", to_np(dv), rv, rule="rounded")


# Shapes whose 256-key blocks give at least 512 workgroups, so that dK and dV
# come from the pass with 256-key workgroups (32 keys per wave at d = 64, 64 at
# d = 128), and (with O's residual) dQ from the pass with 256-row workgroups (64
# rows per wave at d = 64, 32 at d = 128); smaller grids take the passes with
# 128-row workgroups, which the tests above cover: ragged lengths, both masks,
# d = 64 and 128, shared K/V heads, and fewer query rows than keys.
WIDE_GRID = [(2, 256, 256, 300, 300, 128), (1, 512, 512, 65, 65, 64), (4, 256, 128, 257, 257, 128),
             (1, 512, 256, 100, 333, 128), (2, 256, 256, 700, 700, 64), (2, 512, 256, 300, 300, 64),
             (1, 1024, 512, 200, 333, 64)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d", WIDE_GRID)
def test_bf16_backward_wide_grid_passes(fa, B, H, Hkv, Nq, Nk, d, causal):
    import torch
    assert ((Nk + 255) // 256) * B * Hkv >= 512
    say(f"fa_bwd_rect (256-key workgroups) B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} "
        f"causal={causal} seed=25")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, d, seed=25, with_do=True)
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    q64, k64, v64, do64 = inp.as_float64()
    with single_threaded_blas():
        rq, rk, rv = ora.rect_bwd(q64, k64, v64, do64, causal, scale, workers=oracle_workers())
    for mode in MODES:
        say(f"  D from {mode}")
        o_res = torch.empty_like(q) if mode == "o_res" else None
        o, lse = fa.fa_fwd_rect(q, k, v, causal=causal, scale=scale, o_res=o_res)
        dq, dk, dv = fa.fa_bwd_rect(q, k, v, o, do, lse, causal=causal, scale=scale,
                                    o_res=o_res)
        torch.cuda.synchronize()
        check_bf16(f"dQ ({mode})", to_np(dq), rq)
        check_bf16(f"dK ({mode})", to_np(dk), rk)
        check_bf16(f"dV ({mode})", to_np(dv), rv)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bf16_backward_wide_grid_stress(fa, causal):
    """The stress inputs (q, k x3, values of mean 32) on a grid wide enough for
    the 64-row passes, D from O and its residual: every element, "rounded"
    rule."""
    B, H, N, d = 1, 128, 1024, 128
    assert ((N + 255) // 256) * B * H >= 512
    say(f"fa_bwd wide-grid stress B={B} H={H} N={N} d={d} causal={causal} v_mean=32 seed=26")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=26, qk_mult=3.0, with_do=True, v_mean=32.0)
    scale = float(np.float32(1 / np.sqrt(d)))
    dq, dk, dv = _gpu_fwd_bwd(fa, inp, causal, scale, "o_res")
    q64, k64, v64, do64 = inp.as_float64()
    with single_threaded_blas():
        rq, rk, rv = ora.attention_bwd(q64, k64, v64, do64, causal, scale,
                                       workers=oracle_workers())
    check_bf16("dQ", to_np(dq), rq, rule="rounded")
    check_bf16("dK", to_np(dk), rk, rule="rounded")
    check_bf16("dV", to_np(dv), rv, rule="rounded")


def test_backward_phases_equal_fa_bwd(fa):
    """fa_bwd is exactly its three phases, and repeated calls give equal bits."""
    import torch
    B, H, N, d, causal = 2, 2, 333, 128, True
    say(f"fa_bwd phases B={B} H={H} N={N} d={d} causal={causal} seed=23")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=23, with_do=True)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    dq1, dk1, dv1 = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    dq2, dk2, dv2 = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=q.device)
    dq3, dk3, dv3 = (torch.empty_like(q) for _ in range(3))
    fa.fa_bwd_preprocess(q, k, v, o, do, ws)
    fa.fa_bwd_dq(q, k, v, do, lse, ws, dq3, causal=causal)
    fa.fa_bwd_dkdv(q, k, v, do, ws, dk3, dv3, causal=causal)
    torch.cuda.synchronize()
    for a, b, c in ((dq1, dq2, dq3), (dk1, dk2, dk3), (dv1, dv2, dv3)):
        assert torch.equal(a, b) and torch.equal(a, c)
    # the same with O's residual (D from the preprocess)
    o_res = torch.empty_like(q)
    o2, lse2 = fa.fa_fwd(q, k, v, causal=causal, o_res=o_res)
    assert torch.equal(o2, o) and torch.equal(lse2, lse)   # the residual changes nothing else
    dq1, dk1, dv1 = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, o_res=o_res)
    dq2, dk2, dv2 = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, o_res=o_res)
    fa.fa_bwd_preprocess(q, k, v, o, do, ws, o_res=o_res)
    fa.fa_bwd_dq(q, k, v, do, lse, ws, dq3, causal=causal, d_ready=True)
    fa.fa_bwd_dkdv(q, k, v, do, ws, dk3, dv3, causal=causal)
    torch.cuda.synchronize()
    for a, b, c in ((dq1, dq2, dq3), (dk1, dk2, dk3), (dv1, dv2, dv3)):
        assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("B,H,N,d", [(1, 64, 2048, 128), (1, 32, 1024, 256)])
def test_backward_phases_wide_grid_equal_fa_bwd(fa, B, H, N, d):
    """At grids where both matrix passes have 16-row steps (the dQ pass then
    writes the fp16 Q and dO rows of the dK/dV pass), the three phases with
    O's residual are exactly fa_bwd with it, and repeated calls are equal."""
    import torch
    causal = True
    say(f"fa_bwd phases wide grid B={B} H={H} N={N} d={d} causal seed=29")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=29, with_do=True)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    o_res = torch.empty_like(q)
    o, lse = fa.fa_fwd(q, k, v, causal=causal, o_res=o_res)
    dq1, dk1, dv1 = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, o_res=o_res)
    dq2, dk2, dv2 = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, o_res=o_res)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=q.device)
    dq3, dk3, dv3 = (torch.empty_like(q) for _ in range(3))
    fa.fa_bwd_preprocess(q, k, v, o, do, ws, o_res=o_res)
    fa.fa_bwd_dq(q, k, v, do, lse, ws, dq3, causal=causal, d_ready=True)
    fa.fa_bwd_dkdv(q, k, v, do, ws, dk3, dv3, causal=causal)
    torch.cuda.synchronize()
    for a, b, c in ((dq1, dq2, dq3), (dk1, dk2, dk3), (dv1, dv2, dv3)):
        assert torch.equal(a, b) and torch.equal(a, c)
