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

EPS_MMA is an accuracy requirement placed on the matrix core, not a
measurement of it. The products of two e4m3 values are exact (8 significant
bits). A d-term sum formed in fp32, in any order, is within
gamma_d = d 2^-24 / (1 - d 2^-24) of sum |a b| (about 2^-17 at d = 128). The
matrix core's order and width of addition are not specified, and narrower
accumulators exist (sums aligned to the largest term and truncated). The
model therefore admits 16 times the fp32 bound: EPS_MMA = 2^-13, which
allows about 18 significant bits in the sums.

The element-wise bound above is a worst case and cannot tell a coarser
rounding from e4m3: the worst case of e5m2 probabilities (2 fraction bits) is
only twice e4m3's, and the bound holds margin for the tails. The error's
distribution can tell them apart. Treat each rounding error as uniform over
at most [-w_ij, w_ij]. Add the bf16 rounding of O as uniform over
[-ulp, ulp], twice its real width, so that rows whose error is mostly that
rounding stay well below the limit. Then
  sigma_ic^2 = sum_j (w_ij^2 / 3)(v_jc - o_ic)^2 / (sum_j pi_ij)^2
               + ulp_bf16(o_ic)^2 / 3
bounds the variance of element (i, c). The root mean square of
(o~ - o) / sigma over a set of outputs is then at most about 1. A plain
simulation of the e4m3 arithmetic gives 0.63-0.75 (w over-states the
rounding of values inside a binade). With e5m2 probabilities it gives
1.14-1.57. check_fp8_rms requires at most RMS_LIMIT = 1.
"""
from __future__ import annotations

import numpy as np

U8 = 2.0 ** -4          # e4m3 unit roundoff (3 fraction bits)
W_ABS = 2.0 ** -14      # half the e4m3 subnormal spacing 2^-9, over the 2^4 scale
EPS_MMA = 2.0 ** -13
RMS_LIMIT = 1.0


def _bf16_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def row_tolerance(q, k, v, qpos, causal, scale, o_ref):
    """Tolerances for query rows q [R, d] at sequence positions qpos [R]
    against keys k, v [Nk, d], given the exact outputs o_ref [R, d] (the
    oracle's). Returns (tol_o [R, d], tol_lse [R], sigma_o [R, d]): the
    element-wise bounds and the standard deviation bound of the module
    docstring."""
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
    P = np.sum(pi, axis=1)
    tol = np.zeros_like(o_ref)
    sigma = np.zeros_like(o_ref)
    for i in range(R):
        ulp = _bf16_ulp(o_ref[i])
        if not np.any(valid[i]) or D[i] <= 0:
            tol[i] = ulp
            sigma[i] = ulp / np.sqrt(3.0)
            continue
        dv = np.abs(v - o_ref[i][None, :])                       # [Nk, d]
        var = (w[i] ** 2 / 3.0) @ (dv ** 2)
        worst = (w[i] @ dv) / D[i]
        stat = 6.0 * np.sqrt(var) / D[i]
        score = 2.0 * E[i] * (pi[i] @ dv) / D[i]
        acc = (EPS_MMA + 2.0 ** -24 * Nk / 64) * (pi[i] @ np.abs(v)) / D[i]
        tol[i] = np.minimum(worst, stat) + score + acc + ulp
        sigma[i] = np.sqrt(var / P[i] ** 2 + ulp ** 2 / 3.0)
    tol_lse = 1e-3 + E + 2.0 ** -24 * Nk
    return tol, tol_lse, sigma


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


def check_fp8_rms(name, gpu, ref, sigma, say=print, limit=RMS_LIMIT):
    """Root mean square of (gpu - ref) / sigma over all elements <= limit
    (the distribution check of the module docstring); returns it."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape == sigma.shape, (name, gpu.shape, ref.shape, sigma.shape)
    z = (gpu - ref) / sigma
    rms = float(np.sqrt(np.mean(z * z)))
    say(f"  {name}: rms((gpu - oracle) / sigma) = {rms:.3f} (limit {limit:g}) n={z.size}")
    assert rms <= limit, f"{name}: error rms {rms:.3f} sigma > {limit:g}: coarser than e4m3"
    return rms
