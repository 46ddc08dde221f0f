"""fp64 CPU oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE. Only the tests, the package entry's smoke check and the
benchmark's CPU-baseline leg may import or run anything in ``oracle/``. The
HIP library never calls it and shares no code with it.

What it computes is the plain definition, written out and materialised:

  forward ("FlashAttention" page, systems-analysis.ru, section "Problem of
  standard attention"): per batch entry b and head h,
      S   = scale * Q K^T                      (N x N)
      S_ij = -inf for j > i                    (causal mask; the section
                                                "Fusing into one CUDA kernel"
                                                lists masking among the fused
                                                steps, the lower-triangular
                                                shape is the plainest reading)
      m_i = max_j S_ij
      P   = exp(S - m) / sum_j exp(S - m)      (row softmax)
      O   = P V
      lse_i = m_i + ln sum_j exp(S_ij - m_i)   (natural-log logsumexp: the two
                                                statistics that the section
                                                "Online softmax" keeps, max and
                                                exp-sum, combined)

  backward (the pages only imply training, "FlashAttention-2" page,
  section "Performance"; the gradients are textbook calculus of the forward
  for the scalar loss L = sum(O * dO)):
      dV = P^T dO
      dP = dO V^T
      D_i = sum_j P_ij dP_ij
      dS = P * (dP - D)
      dQ = scale * dS K
      dK = scale * dS^T Q

Each query row's softmax only depends on that row, so rows are processed in
blocks of at most ``ROW_BLOCK`` rows; within a block S and P are fully
materialised. This is still the one-shot definition, not an online softmax.

Arrays are float64 numpy arrays of shape [B, H, N, d]; lse is [B, H, N].
A row with every key masked (impossible for the square causal case) gets
O = 0 and lse = -inf.

Shared K/V heads (the "FlashAttention" page, section "FlashAttention-2
(2023)", names multi-query attention among the extensions; grouped heads are
the plainest generalisation): k and v may have Hkv heads, Hkv dividing H, and
query head h then uses K/V head h // (H // Hkv). Each query head's forward is
the definition above with that K/V head; the gradient of a shared K/V head is
the sum of its query heads' gradients (the chain rule through a shared input).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

ROW_BLOCK = 1024


def _scores(q_rows: np.ndarray, k: np.ndarray, rows: np.ndarray,
            causal: bool, scale: float) -> np.ndarray:
    """scale * Q_rows K^T with the causal mask applied (-inf where j > i)."""
    s = scale * (q_rows @ k.T)
    if causal:
        j = np.arange(k.shape[0])
        s = np.where(j[None, :] > rows[:, None], -np.inf, s)
    return s


def _softmax_rows(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row softmax P and natural-log logsumexp of a score block."""
    m = np.max(s, axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = np.sum(e, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(l[:, None] > 0, e / l[:, None], 0.0)
        lse = np.where(l > 0, m_safe + np.log(l), -np.inf)
    return p, lse


def head_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
             scale: float, rows: Optional[np.ndarray] = None, pos0: int = 0
             ) -> Tuple[np.ndarray, np.ndarray]:
    """Forward for one (b, h) head: q [Nq, d] (rows selected), k, v [Nk, d].

    Query row i sits at sequence position pos0 + i: with ``causal`` it keeps
    the keys j <= pos0 + i (pos0 = 0: the square, top-left aligned case)."""
    n = q.shape[0]
    if rows is None:
        rows = np.arange(n)
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    for r0 in range(0, len(rows), ROW_BLOCK):
        rr = rows[r0:r0 + ROW_BLOCK]
        s = _scores(q[rr], k, rr + pos0, causal, scale)
        p, ls = _softmax_rows(s)
        o[r0:r0 + len(rr)] = p @ v
        lse[r0:r0 + len(rr)] = ls
    return o, lse


def head_probs(q: np.ndarray, k: np.ndarray, causal: bool, scale: float) -> np.ndarray:
    """The full probability matrix P = softmax(scale Q K^T) of one head."""
    rows = np.arange(q.shape[0])
    p, _ = _softmax_rows(_scores(q, k, rows, causal, scale))
    return p


def head_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
             causal: bool, scale: float, pos0: int = 0
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Backward for one head: q, do [Nq, d], k, v [Nk, d]; returns (dq, dk, dv)
    shaped like q, k, v. Query row i sits at position pos0 + i as in head_fwd
    (a row that keeps no key has P = 0 and contributes nothing)."""
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, ROW_BLOCK):
        rr = np.arange(r0, min(n, r0 + ROW_BLOCK))
        p, _ = _softmax_rows(_scores(q[rr], k, rr + pos0, causal, scale))
        dv += p.T @ do[rr]
        dp = do[rr] @ v.T
        dsum = np.sum(p * dp, axis=1)
        ds = p * (dp - dsum[:, None])
        dq[rr] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rr])
    return dq, dk, dv


def head_dq_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                 causal: bool, scale: float, rows: np.ndarray, pos0: int = 0) -> np.ndarray:
    """dQ of selected query rows of one head (the backward formulas above,
    restricted to those rows: row i of dQ only needs row i of P and dP).
    Query row i sits at position pos0 + i as in head_fwd."""
    rows = np.asarray(rows)
    dq = np.zeros((len(rows), q.shape[1]))
    for r0 in range(0, len(rows), ROW_BLOCK):
        rr = rows[r0:r0 + ROW_BLOCK]
        p, _ = _softmax_rows(_scores(q[rr], k, rr + pos0, causal, scale))
        dp = do[rr] @ v.T
        dsum = np.sum(p * dp, axis=1)
        ds = p * (dp - dsum[:, None])
        dq[r0:r0 + len(rr)] = scale * (ds @ k)
    return dq


def _group(H: int, k: np.ndarray) -> int:
    """Query heads per K/V head (k has shape [B, Hkv, N, d], Hkv dividing H)."""
    Hkv = k.shape[1]
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{Hkv} K/V heads do not divide {H} query heads")
    return H // Hkv


def _heads(B: int, H: int, heads: Optional[Iterable[Tuple[int, int]]]):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def _pool_map(fn, items, workers: Optional[int]):
    workers = workers or len(os.sched_getaffinity(0))
    if workers <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
                  scale: float, heads: Optional[Sequence[Tuple[int, int]]] = None,
                  rows: Optional[np.ndarray] = None, workers: Optional[int] = 1
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Forward over [B, H, N, d] arrays.

    ``heads`` restricts the work to a list of (b, h) pairs and ``rows`` to a
    sorted set of query rows; the result then has shape
    [len(heads), len(rows), d] (and [len(heads), len(rows)] for lse).
    Without either, the result has the input's [B, H, N, d] shape.
    """
    B, H, N, d = q.shape
    G = _group(H, k)
    hs = _heads(B, H, heads)
    rr = np.arange(N) if rows is None else np.asarray(rows)

    def one(bh):
        b, h = bh
        return head_fwd(q[b, h], k[b, h // G], v[b, h // G], causal, scale, rr)

    res = _pool_map(one, hs, workers)
    o = np.stack([r[0] for r in res]) if res else np.zeros((0, len(rr), v.shape[-1]))
    lse = np.stack([r[1] for r in res]) if res else np.zeros((0, len(rr)))
    if heads is None and rows is None:
        return o.reshape(B, H, N, v.shape[-1]), lse.reshape(B, H, N)
    return o, lse


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                  causal: bool, scale: float,
                  heads: Optional[Sequence[Tuple[int, int]]] = None,
                  workers: Optional[int] = 1):
    """Backward over [B, H, N, d] arrays (k, v: [B, Hkv, N, d]).

    Without ``heads``: dQ [B, H, N, d] and dK, dV [B, Hkv, N, d], a shared
    K/V head's gradient being the sum over its query heads. With ``heads`` (a
    list of query heads (b, h)): each listed query head's own dQ, dK, dV
    contributions, stacked, before any summing.
    """
    B, H, N, d = q.shape
    G = _group(H, k)
    hs = _heads(B, H, heads)

    def one(bh):
        b, h = bh
        return head_bwd(q[b, h], k[b, h // G], v[b, h // G], do[b, h], causal, scale)

    res = _pool_map(one, hs, workers)
    dq = np.stack([r[0] for r in res])
    dk = np.stack([r[1] for r in res])
    dv = np.stack([r[2] for r in res])
    if heads is None:
        kv_shape = (B, H // G, G, N, d)
        return (dq.reshape(B, H, N, d), dk.reshape(kv_shape).sum(axis=2),
                dv.reshape(kv_shape).sum(axis=2))
    return dq, dk, dv


def rect_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
             heads: Optional[Sequence[Tuple[int, int]]] = None,
             workers: Optional[int] = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of Nq query rows against Nk keys, the queries being the last
    Nq positions: q [B, H, Nq, d], k and v [B, Hkv, Nk, d] (shared heads as for
    attention_fwd). Query row i sits at position Nk - Nq + i, so with
    ``causal`` it keeps the keys j <= Nk - Nq + i (bottom-right alignment;
    when Nq > Nk the first Nq - Nk rows keep none: O = 0, lse = -inf); without,
    every key. Returns O [B, H, Nq, d] and lse [B, H, Nq] (with ``heads``: the
    listed query heads, stacked)."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    G = _group(H, k)
    hs = _heads(B, H, heads)

    def one(bh):
        b, h = bh
        return head_fwd(q[b, h], k[b, h // G], v[b, h // G], causal, scale, pos0=Nk - Nq)

    res = _pool_map(one, hs, workers)
    o = np.stack([r[0] for r in res])
    lse = np.stack([r[1] for r in res])
    if heads is None:
        return o.reshape(B, H, Nq, v.shape[-1]), lse.reshape(B, H, Nq)
    return o, lse


def rect_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, causal: bool,
             scale: float, heads: Optional[Sequence[Tuple[int, int]]] = None,
             workers: Optional[int] = 1):
    """Backward of rect_fwd: q, do [B, H, Nq, d], k, v [B, Hkv, Nk, d], query
    row i at position Nk - Nq + i. Without ``heads``: dQ [B, H, Nq, d] and
    dK, dV [B, Hkv, Nk, d] (a shared K/V head's gradient summed over its query
    heads); with ``heads``: each listed query head's own dQ, dK, dV, stacked,
    before any summing."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    G = _group(H, k)
    hs = _heads(B, H, heads)

    def one(bh):
        b, h = bh
        return head_bwd(q[b, h], k[b, h // G], v[b, h // G], do[b, h], causal, scale,
                        pos0=Nk - Nq)

    res = _pool_map(one, hs, workers)
    dq = np.stack([r[0] for r in res])
    dk = np.stack([r[1] for r in res])
    dv = np.stack([r[2] for r in res])
    if heads is None:
        kv_shape = (B, H // G, G, Nk, d)
        return (dq.reshape(B, H, Nq, d), dk.reshape(kv_shape).sum(axis=2),
                dv.reshape(kv_shape).sum(axis=2))
    return dq, dk, dv


def decode_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
               workers: Optional[int] = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of the last Nq positions of a sequence of Nk >= Nq keys (the
    decoding step of an inference system): q [B, H, Nq, d], k and v
    [B, Hkv, Nk, d] (shared heads as for attention_fwd). Query row i sits at
    position Nk - Nq + i, so with ``causal`` it keeps the keys
    j <= Nk - Nq + i (bottom-right alignment); without, every key. Returns
    O [B, H, Nq, d] and lse [B, H, Nq]."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if Nq > Nk:
        raise ValueError("decoding needs Nq <= Nk")
    G = _group(H, k)

    def one(bh):
        b, h = bh
        return head_fwd(q[b, h], k[b, h // G], v[b, h // G], causal, scale, pos0=Nk - Nq)

    res = _pool_map(one, _heads(B, H, None), workers)
    o = np.stack([r[0] for r in res]).reshape(B, H, Nq, v.shape[-1])
    lse = np.stack([r[1] for r in res]).reshape(B, H, Nq)
    return o, lse


def online_softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                             causal: bool, scale: float,
                             cuts: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of one head by the block-wise ("online") softmax.

    Follows the "FlashAttention" page (systems-analysis.ru), sections "Tiling"
    and "Online softmax": keys and values are taken block by block (block
    boundaries at ``cuts``, any increasing positions in (0, N)); for every
    query row two running statistics are kept, the current maximum m and the
    sum of exponentials l, and both and the unnormalised output are updated as
    each block arrives:

        m'   = max(m, max_j S_blk)
        l    = exp(m - m') l + sum_j exp(S_blk - m')
        acc  = exp(m - m') acc + exp(S_blk - m') V_blk
        m    = m'

    and at the end O = acc / l, lse = m + ln l. This is a model of the
    recurrence that a tiled kernel runs, used to show that splitting at
    arbitrary points gives the one-shot result.
    """
    n, dv = q.shape[0], v.shape[1]
    nk = k.shape[0]
    bounds = [0] + sorted(int(c) for c in cuts) + [nk]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, dv))
    rows = np.arange(n)
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b <= a:
            continue
        s = scale * (q @ k[a:b].T)
        if causal:
            j = np.arange(a, b)
            s = np.where(j[None, :] > rows[:, None], -np.inf, s)
        m_new = np.maximum(m, np.max(s, axis=1))
        m_safe = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - m_safe)           # exp(-inf) = 0 for the first block
        e = np.exp(s - m_safe[:, None])
        l = alpha * l + np.sum(e, axis=1)
        acc = alpha[:, None] * acc + e @ v[a:b]
        m = m_new
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l[:, None] > 0, acc / l[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(l), -np.inf)
    return o, lse
