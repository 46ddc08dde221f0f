"""Error model of the e4m3 forward (fa_fwd_fp8), used as its parity tolerance.

The kernel's arithmetic on the real (dequantised) inputs, per query row i:
  s_ij  = scale q_i.k_j       e4m3 MFMA: exact products, sums with a relative
                              error of at most EPS_MMA of scale sum_k |q_ik k_jk|
  p_ij  = 2^4 exp(s_ij - m_i) fp32; m_i is a reference no higher than the row
                              maximum (it lags by at most 4 log2 units)
  p~_ij = e4m3(p_ij)          round to nearest even: |p~ - p| <= max(2^-4 p, 2^-10)
  o_i   = sum_j p~_ij v_j / sum_j p~_ij     e4m3 MFMA, fp32 accumulation, bf16 store
With the exact weights pi_ij = exp(s_ij - max_j s_ij) and lambda_i = p_ij / pi_ij
(>= 2^4, the same for every j of the row):
  o~_i - o_i = sum_j (p~_ij/lambda_i - pi_ij)(v_j - o_i) / sum_j p~_ij/lambda_i,
and each weight's error is at most w_ij = max(2^-4 pi_ij, 2^-14). With
D_i = sum_j max(0, pi_ij - w_ij) (a lower bound of the denominator):
  worst case   sum_j w_ij |v_jc - o_ic| / D_i
  6 sigma      6 sqrt(sum_j (w_ij^2 / 3)(v_jc - o_ic)^2) / D_i  (rounding errors
               taken as independent and uniform over at most [-w_ij, w_ij])
and the tolerance of element (i, c) is
  min(worst, 6 sigma)
  + 2 E_i sum_j pi_ij |v_jc - o_ic| / D_i        score error, E_i = EPS_MMA max_j
                                                 scale sum_k |q_ik k_jk|
  + (EPS_MMA + 2^-24 Nk / 64) sum_j pi_ij |v_jc| / D_i   accumulation of P V
  + ulp_bf16(o_ic)                               output rounding.
lse comes from the fp32 sum of the unrounded p: its tolerance is
1e-3 + E_i + 2^-24 Nk.

EPS_MMA = 2^-13 is four times the largest relative error (2^-15.8 of
sum |a b|) measured for the 32x32x64 e4m3 product on random operands; the
product is not exact in fp32.
"""
from __future__ import annotations

import numpy as np

U8 = 2.0 ** -4          # e4m3 unit roundoff (3 fraction bits)
W_ABS = 2.0 ** -14      # half the e4m3 subnormal spacing 2^-9, over the 2^4 scale
EPS_MMA = 2.0 ** -13


def _bf16_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def row_tolerance(q, k, v, qpos, causal, scale, o_ref):
    """Tolerances for query rows q [R, d] at sequence positions qpos [R]
    against keys k, v [Nk, d], given the exact outputs o_ref [R, d] (the
    oracle's). Returns (tol_o [R, d], tol_lse [R])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    R, Nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    valid = np.ones((R, Nk), dtype=bool)
    if causal:
        valid = np.arange(Nk)[None, :] <= np.asarray(qpos)[:, None]
    s = np.where(valid, s, -np.inf)
    smax = np.max(s, axis=1, keepdims=True)
    smax = np.where(np.isfinite(smax), smax, 0.0)
    pi = np.where(valid, np.exp(s - smax), 0.0)
    w = np.where(valid, np.maximum(U8 * pi, W_ABS), 0.0)
    D = np.sum(np.maximum(0.0, pi - w), axis=1)
    E = EPS_MMA * scale * np.max(np.where(valid, np.abs(q) @ np.abs(k).T, 0.0), axis=1)
    tol = np.zeros_like(o_ref)
    for i in range(R):
        if not np.any(valid[i]) or D[i] <= 0:
            tol[i] = _bf16_ulp(o_ref[i])
            continue
        dv = np.abs(v - o_ref[i][None, :])                       # [Nk, d]
        worst = (w[i] @ dv) / D[i]
        stat = 6.0 * np.sqrt((w[i] ** 2 / 3.0) @ (dv ** 2)) / D[i]
        score = 2.0 * E[i] * (pi[i] @ dv) / D[i]
        acc = (EPS_MMA + 2.0 ** -24 * Nk / 64) * (pi[i] @ np.abs(v)) / D[i]
        tol[i] = np.minimum(worst, stat) + score + acc + _bf16_ulp(o_ref[i])
    tol_lse = 1e-3 + E + 2.0 ** -24 * Nk
    return tol, tol_lse


def check_fp8(name, gpu, ref, tol, say=print):
    """|gpu - ref| <= tol elementwise; reports the largest error and the
    largest error / tolerance ratio."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape == tol.shape, (name, gpu.shape, ref.shape, tol.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    err = np.abs(gpu - ref)
    ratio = err / tol
    say(f"  {name}: max_abs={err.max():.3e} max_tol={tol.max():.3e} "
        f"median_tol={np.median(tol):.3e} max_err/tol={ratio.max():.3f} n={err.size}")
    bad = err > tol
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {int(bad.sum())} elements out of tolerance; first "
                             f"{idx.tolist()} gpu={gpu[bad][:5]} ref={ref[bad][:5]} "
                             f"tol={tol[bad][:5]}")
    return float(ratio.max())
