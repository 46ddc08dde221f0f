"""Parity of the e4m3 forward (fa_fwd_fp8) against the fp64 oracle evaluated on
the dequantised inputs (descale * e4m3 value, exact in float64), through the
C ABI, with the tolerance of the fp8 error model in fp8_tolerance.py.

Small shapes (several tiles, ragged tails, Nq != Nk with bottom-right causal
alignment and rows that see no key, shared K/V heads, a sharpened softmax)
are compared on every element; the benchmark workloads on sampled rows of
every head.
"""
import concurrent.futures as cf

import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import record_model_check, say, sample_rows, to_np
import fp8_tolerance as ft

pytestmark = pytest.mark.gpu

D = 128


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
    q, k, v = (wl.fp8_to_device(x) for x in (inp.q8, inp.k8, inp.v8))
    o, lse = fa.fa_fwd_fp8(q, k, v, inp.dq, inp.dk, inp.dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


def _check_rows(name, o, lse, ro, rl, q64, k64, v64, pairs, rows, Nq, Nk, causal, scale, G):
    """o, lse, ro, rl: [len(pairs), R, ...] for query rows `rows` of the listed
    (b, h); tolerance row by row from the error model."""
    qpos = np.asarray(rows) + (Nk - Nq)

    def one(i):
        b, h = pairs[i]
        return ft.row_tolerance(q64[b, h][rows], k64[b, h // G], v64[b, h // G], qpos, causal,
                                scale, ro[i])

    with cf.ThreadPoolExecutor(8) as ex:
        res = list(ex.map(one, range(len(pairs))))
    tol = np.stack([r[0] for r in res])
    tol_lse = np.stack([r[1] for r in res])
    sigma = np.stack([r[2] for r in res])
    err_o = np.abs(np.asarray(o, np.float64) - ro)
    record_model_check(f"O {name}", err_o, tol, bool(np.all(err_o <= tol)))
    ft.check_fp8(f"O {name}", o, ro, tol, say=say)
    rms = float(np.sqrt(np.mean(((np.asarray(o, np.float64) - ro) / sigma) ** 2)))
    record_model_check(f"O {name}: rms of error / sigma", np.array([rms]),
                       np.array([ft.RMS_LIMIT]), rms <= ft.RMS_LIMIT)
    ft.check_fp8_rms(f"O {name}", o, ro, sigma, say=say)
    both_inf = np.isneginf(lse) & np.isneginf(rl)
    err = np.where(both_inf, 0.0, np.abs(lse - rl))
    record_model_check(f"lse {name}", err, np.broadcast_to(tol_lse, err.shape),
                       bool(np.all(np.isfinite(err)) and np.all(err <= tol_lse)))
    say(f"  lse {name}: max_abs={np.nanmax(err):.3e} max_tol={tol_lse.max():.3e}")
    assert np.all(np.isfinite(err)) and np.all(err <= tol_lse)


SMALL = [(1, 2, 2, 300, 300), (2, 4, 2, 129, 129), (1, 2, 1, 200, 517), (1, 2, 1, 300, 100),
         (1, 1, 1, 1, 1), (1, 3, 3, 520, 520)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk", SMALL)
def test_fp8_forward_small(fa, B, H, Hkv, Nq, Nk, causal):
    say(f"fa_fwd_fp8 B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={D} causal={causal} seed=101")
    inp = wl.make_fp8_inputs(B, H, Hkv, Nq, Nk, D, seed=101)
    scale = float(np.float32(1 / np.sqrt(D)))
    o, lse = _run(fa, inp, causal, scale)
    q64, k64, v64 = inp.as_float64()
    ro, rl = ora.rect_fwd(q64, k64, v64, causal, scale, workers=None)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    rows = np.arange(Nq)
    _check_rows("(every element)", o.reshape(B * H, Nq, D), lse.reshape(B * H, Nq),
                ro.reshape(B * H, Nq, D), rl.reshape(B * H, Nq), q64, k64, v64, pairs, rows,
                Nq, Nk, causal, scale, H // Hkv)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_fp8_forward_sharp_softmax(fa, causal):
    """q and k drawn 3x wider before quantisation: sharper rows, later tiles
    moving the reference maximum."""
    B, H, N = 1, 4, 640
    say(f"fa_fwd_fp8 sharpened B={B} H={H} N={N} causal={causal} seed=102")
    inp = wl.make_fp8_inputs(B, H, H, N, N, D, seed=102, qk_mult=3.0)
    scale = float(np.float32(1 / np.sqrt(D)))
    o, lse = _run(fa, inp, causal, scale)
    q64, k64, v64 = inp.as_float64()
    ro, rl = ora.rect_fwd(q64, k64, v64, causal, scale, workers=None)
    pairs = [(0, h) for h in range(H)]
    _check_rows("(every element)", o[0], lse[0], ro[0], rl[0], q64, k64, v64, pairs,
                np.arange(N), N, N, causal, scale, 1)


@pytest.mark.parametrize("name", list(wl.FP8_WORKLOADS))
def test_fp8_forward_workload(fa, name):
    """The benchmark workloads in the benchmark's launch: sampled rows of every
    head."""
    w = wl.FP8_WORKLOADS[name]
    say(f"fp8 workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    inp = wl.make_fp8_inputs(w.B, w.H, w.H, w.N, w.N, w.d, w.seed)
    o, lse = _run(fa, inp, w.causal, w.scale)
    q64, k64, v64 = inp.as_float64()
    rows = sample_rows(w.N, 24, seed=w.seed)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    ro, rl = ora.attention_fwd(q64, k64, v64, w.causal, w.scale, heads=pairs, rows=rows,
                               workers=None)
    _check_rows("(sampled rows, all heads)", o.reshape(w.B * w.H, w.N, w.d)[:, rows],
                lse.reshape(w.B * w.H, w.N)[:, rows], ro, rl, q64, k64, v64, pairs, rows, w.N,
                w.N, w.causal, w.scale, 1)
