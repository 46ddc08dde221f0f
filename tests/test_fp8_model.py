"""CPU pins of the fp8 path's test infrastructure: the e4m3 codec of the input
generator against the format's definition, and the fp8 error model
(fp8_tolerance) against a plain simulation of the kernel's arithmetic."""
import math

import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
import fp8_tolerance as ft


def _e4m3_value(b: int) -> float:
    """OCP e4m3 (OFP8 "E4M3"): sign, 4 exponent bits (bias 7), 3 mantissa bits;
    exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities."""
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return math.nan
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_e4m3_decode_matches_the_format_definition():
    codes = np.arange(256, dtype=np.uint8)
    got = wl.e4m3_decode(codes)
    want = np.array([_e4m3_value(int(b)) for b in codes])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert want[0x7E] == 448.0 and want[0x01] == 2.0 ** -9 and want[0x38] == 1.0


def test_e4m3_encode_round_trips_and_rounds_to_nearest_even():
    codes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    vals = wl.e4m3_decode(codes).astype(np.float32)
    back = wl.e4m3_encode(vals)
    # -0 and +0 both exist; everything else must round-trip
    assert np.array_equal(back, codes)
    # ties go to the even mantissa; halfway to the smallest subnormal goes to 0
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 440.0], np.float32)
    got = wl.e4m3_decode(wl.e4m3_encode(x))
    assert got.tolist() == [1.0, 1.25, 0.0, 2.0 ** -8, 448.0]


def test_quantize_e4m3_uses_the_full_range():
    r = np.random.default_rng(5)
    x = r.standard_normal(1000).astype(np.float32)
    b, s = wl.quantize_e4m3(x)
    y = wl.e4m3_decode(b) * s
    assert np.max(np.abs(wl.e4m3_decode(b))) == 448.0
    assert np.max(np.abs(y - x) / np.maximum(np.abs(x), 2.0 ** -6 * s)) <= 2.0 ** -4 + 1e-6


def _simulate(q, k, v, qpos, causal, scale, rng, fmt="e4m3"):
    """The kernel's arithmetic in numpy: a lagging reference at most 4 log2
    units below the row maximum, p = 2^4 exp(s - m), p rounded to the 8-bit
    format, O normalised by the sum of the rounded p; lse from the unrounded
    sum."""
    import torch
    s = scale * (q @ k.T)
    valid = np.arange(k.shape[0])[None, :] <= qpos[:, None] if causal else np.ones(s.shape, bool)
    s = np.where(valid, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True) - rng.uniform(0, 4 * math.log(2), (s.shape[0], 1))
    p = (16.0 * np.exp(s - m)).astype(np.float32)
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    pq = torch.from_numpy(p).to(dt).to(torch.float64).numpy()
    o = (pq @ v) / pq.sum(axis=1, keepdims=True)
    lse = np.log(p.astype(np.float64).sum(axis=1)) + m[:, 0] - math.log(16.0)
    return o, lse


CASES = [(1, 40, 64, False, 1.0), (2, 100, 300, True, 1.0), (3, 64, 64, True, 3.0),
         (4, 17, 1000, False, 1.0)]


@pytest.mark.parametrize("seed,Nq,Nk,causal,mult", CASES)
def test_error_model_covers_simulated_fp8_arithmetic(seed, Nq, Nk, causal, mult):
    d = 32
    inp = wl.make_fp8_inputs(1, 1, 1, Nq, Nk, d, seed, qk_mult=mult)
    q, k, v = (x[0, 0] for x in inp.as_float64())
    scale = 1 / math.sqrt(d)
    qpos = np.arange(Nq) + (Nk - Nq)
    o_ref, lse_ref = ora.rect_fwd(q[None, None], k[None, None], v[None, None], causal, scale)
    o_ref, lse_ref = o_ref[0, 0], lse_ref[0, 0]
    tol, tol_lse, sigma = ft.row_tolerance(q, k, v, qpos, causal, scale, o_ref)
    o_sim, lse_sim = _simulate(q, k, v, qpos, causal, scale, np.random.default_rng(seed))
    o_sim = wl.bf16_round(o_sim.astype(np.float32)).astype(np.float64)   # the bf16 store
    ft.check_fp8("O (simulated e4m3)", o_sim, o_ref, tol)
    rms = ft.check_fp8_rms("O (simulated e4m3)", o_sim, o_ref, sigma)
    assert rms >= 0.5      # the model is a bound, but not a loose one
    assert np.all(np.abs(lse_sim - lse_ref) <= tol_lse)


@pytest.mark.parametrize("mistake", ["key_order", "no_v_factor", "lse_shift", "e5m2"])
def test_error_model_rejects_planted_mistakes(mistake):
    """Mistakes a kernel could make leave the tolerance: the V^T key order
    out of step with the probabilities' (adjacent 4-key groups swapped), the
    V factor left out of O, lse without the 2^4 probability scale taken out,
    or probabilities rounded to e5m2 instead of e4m3. e5m2 stays inside the
    element-wise bound (0.65-0.9 of it) but not the distribution check: its
    errors are twice as wide."""
    d, Nq, Nk = 32, 64, 256
    inp = wl.make_fp8_inputs(1, 1, 1, Nq, Nk, d, 9)
    q, k, v = (x[0, 0] for x in inp.as_float64())
    scale = 1 / math.sqrt(d)
    qpos = np.arange(Nq) + (Nk - Nq)
    o_ref, lse_ref = ora.rect_fwd(q[None, None], k[None, None], v[None, None], False, scale)
    o_ref, lse_ref = o_ref[0, 0], lse_ref[0, 0]
    tol, tol_lse, sigma = ft.row_tolerance(q, k, v, qpos, False, scale, o_ref)
    vv = v[np.arange(Nk) ^ 4] if mistake == "key_order" else v
    fmt = "e5m2" if mistake == "e5m2" else "e4m3"
    o_sim, lse_sim = _simulate(q, k, vv, qpos, False, scale, np.random.default_rng(9), fmt)
    o_sim = wl.bf16_round(o_sim.astype(np.float32)).astype(np.float64)
    if mistake == "no_v_factor":
        o_sim = o_sim / inp.dv
    if mistake == "lse_shift":
        lse_sim = lse_sim + math.log(16.0)
        assert np.any(np.abs(lse_sim - lse_ref) > tol_lse)
        return
    if mistake == "e5m2":
        ft.check_fp8("O (e5m2 probabilities)", o_sim, o_ref, tol)   # inside the worst case
        with pytest.raises(AssertionError):
            ft.check_fp8_rms("O (e5m2 probabilities)", o_sim, o_ref, sigma)
        return
    with pytest.raises(AssertionError):
        ft.check_fp8("O (planted mistake)", o_sim, o_ref, tol)
