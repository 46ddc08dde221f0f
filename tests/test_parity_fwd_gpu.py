"""Forward parity: libfa.so (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element on every output; they span
several tiles and a ragged tail. The five full-size workloads run in exactly
the launch configuration the benchmark times and are compared on every
element of every head (the oracle runs over all heads on the host's cores).
"""
import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import (F32_ATOL, LSE_ATOL, check_abs, check_bf16, oracle_workers, say,
                         single_threaded_blas, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    from exact_attention_41_amd import _lib
    _lib.load()
    return fa


def _run_bf16(fa, inp, causal, scale):
    import torch
    q, k, v = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


SMALL = [(1, 1, 1, 64), (1, 1, 17, 128), (2, 3, 64, 64), (1, 2, 65, 128), (2, 2, 300, 64),
         (1, 3, 300, 128), (1, 1, 513, 128), (1, 2, 1000, 64), (3, 1, 700, 128)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,N,d", SMALL)
def test_bf16_forward_small(fa, B, H, N, d, causal):
    say(f"fa_fwd bf16 B={B} H={H} N={N} d={d} causal={causal} seed=11")
    inp = wl.make_inputs(B, H, N, d, "bf16", seed=11)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run_bf16(fa, inp, causal, scale)
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.attention_fwd(q64, k64, v64, causal, scale, workers=None)
    check_bf16("O", to_np(o), ro)
    check_abs("lse", to_np(lse), rl, LSE_ATOL)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,N,d", [(1, 1, 256, 64), (1, 1, 256, 128), (2, 2, 97, 64),
                                     (1, 2, 333, 128)])
def test_f32_forward(fa, B, H, N, d, causal):
    import torch
    say(f"fa_fwd_f32 B={B} H={H} N={N} d={d} causal={causal} seed=12")
    inp = wl.make_inputs(B, H, N, d, "f32", seed=12)
    q, k, v = (wl.to_device(x, "f32") for x in (inp.q, inp.k, inp.v))
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = fa.fa_fwd_f32(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.attention_fwd(q64, k64, v64, causal, scale, workers=None)
    check_abs("O", to_np(o), ro, F32_ATOL)
    check_abs("lse", to_np(lse), rl, LSE_ATOL)


def test_f32_workload_full(fa):
    """The fp32 workload B=1 H=1 N=256 d=64, every output element."""
    import torch
    w = wl.WORKLOADS["fp32_b1h1n256d64"]
    say(f"fa_fwd_f32 workload {w.name}")
    inp = wl.workload_inputs(w)
    q, k, v = (wl.to_device(x, "f32") for x in (inp.q, inp.k, inp.v))
    o, lse = fa.fa_fwd_f32(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.attention_fwd(q64, k64, v64, w.causal, w.scale)
    check_abs("O", to_np(o), ro, F32_ATOL)
    check_abs("lse", to_np(lse), rl, LSE_ATOL)


FULL = ["bf16_b8h16n2048d64", "bf16_b8h16n2048d64_causal", "bf16_b2h32n8192d128_causal_x3",
        "bf16_b1h16n16384d128_causal", "bf16_b4h16n4096d128_causal_bwd"]


@pytest.mark.parametrize("name", FULL)
def test_bf16_forward_workload_full(fa, name):
    """A full-size workload, every element of O and lse."""
    import torch
    w = wl.WORKLOADS[name]
    say(f"fa_fwd workload {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} seed={w.seed}")
    inp = wl.workload_inputs(w)
    o, lse = _run_bf16(fa, inp, w.causal, w.scale)
    q64, k64, v64 = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    say(f"  oracle on {oracle_workers()} threads")
    with single_threaded_blas():
        ro, rl = ora.attention_fwd(q64, k64, v64, w.causal, w.scale, workers=oracle_workers())
    check_bf16(f"O {name}", to_np(o), ro)
    check_abs(f"lse {name}", to_np(lse), rl, LSE_ATOL)
    # Properties over every row: finite output, each row a convex combination
    # of value rows (within bf16 rounding), lse above the diagonal logit bound.
    o_all = o.float()
    assert torch.isfinite(o_all).all() and torch.isfinite(lse).all()
    vmax = torch.from_numpy(inp.v).to(o.device).amax(dim=2, keepdim=True)
    vmin = torch.from_numpy(inp.v).to(o.device).amin(dim=2, keepdim=True)
    assert bool((o_all <= vmax + 1e-2 + 1e-2 * vmax.abs()).all())
    assert bool((o_all >= vmin - 1e-2 - 1e-2 * vmin.abs()).all())
