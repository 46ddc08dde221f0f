"""Helpers shared by the GPU parity tests (tolerances, sampling, device copies).

Tolerances (max-abs, against the fp64 oracle):
  * bf16 O, dQ, dK, dV: an element passes when |gpu - oracle| <= max(1e-2,
    ulp_bf16(|oracle|)). For |x| >= 4 one bf16 ulp is 2^-5 > 1e-2, so even the
    correctly rounded oracle can miss a plain 1e-2 there; the plain max-abs
    error, the rounding floor max|bf16(oracle) - oracle| and the number of
    elements that pass only through the ulp clause are always reported.
  * fp32 O: 1e-5 plain max-abs.
  * logsumexp: 1e-3 plain max-abs.
"""
from __future__ import annotations

import sys

import numpy as np

from exact_attention_41_amd import workloads as wl

BF16_ATOL = 1e-2
F32_ATOL = 1e-5
LSE_ATOL = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_bf16(name: str, gpu: np.ndarray, ref: np.ndarray, atol: float = BF16_ATOL) -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    err = np.abs(gpu - ref)
    bound = np.maximum(atol, bf16_ulp(ref))
    floor = np.abs(wl.bf16_round(ref.astype(np.float32)).astype(np.float64) - ref)
    stats = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "floor": float(floor.max()) if floor.size else 0.0,
        "ulp_clause_only": int(np.sum((err > atol) & (err <= bound))),
        "n": int(err.size),
    }
    say(f"  {name}: max_abs={stats['max_abs']:.3e} bf16_floor={stats['floor']:.3e} "
        f"ulp_only={stats['ulp_clause_only']} n={stats['n']}")
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {int(bad.sum())} elements out of tolerance; first "
                             f"{idx.tolist()} gpu={gpu[bad][:5]} ref={ref[bad][:5]}")
    return stats


def check_abs(name: str, gpu: np.ndarray, ref: np.ndarray, atol: float) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    m = float(np.nanmax(err)) if err.size else 0.0
    say(f"  {name}: max_abs={m:.3e} (tol {atol:g}) n={err.size}")
    assert np.all(np.isfinite(err)), f"{name}: non-finite mismatch"
    assert m <= atol, f"{name}: max abs error {m} > {atol}"
    return m


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Sorted query rows: both ends, tile boundaries and random rows."""
    fixed = [0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 255, 256, 257, 511, 512, N // 2,
             N - 65, N - 64, N - 33, N - 2, N - 1]
    r = np.random.Generator(np.random.PCG64(seed))
    rnd = r.integers(0, N, size=max(0, count - len(fixed)))
    rows = np.unique(np.clip(np.array(fixed + rnd.tolist()), 0, N - 1))
    return rows


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)
