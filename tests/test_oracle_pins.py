"""Pins for the fp64 oracle: each check ties it to something other than itself.

Definition pinned: the "FlashAttention" page (systems-analysis.ru), section
"Problem of standard attention" (softmax(Q K^T / sqrt(d_k)) V); block-wise
exactness from its section "Online softmax"; gradients by finite differences
of the forward (the pages describe no backward).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as ora
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _frac(s):
    return float(Fraction(s))


# --------------------------------------------------------------- golden example
@pytest.mark.parametrize("mask", ["noncausal", "causal"])
def test_hand_worked_example(mask):
    g = json.load(open(os.path.join(GOLDEN, "hand_3keys_d1.json")))
    q, k, v, do = (np.array(g[x], dtype=np.float64)[None, None] for x in ("q", "k", "v", "do"))
    scale = math.log(2.0)
    causal = mask == "causal"
    exp = g[mask]
    o, lse = ora.attention_fwd(q, k, v, causal, scale)
    np.testing.assert_allclose(o[0, 0, :, 0], [_frac(x) for x in exp["o"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], [math.log(_frac(x)) for x in exp["lse_exp"]],
                               rtol=0, atol=1e-14)
    dq, dk, dv = ora.attention_bwd(q, k, v, do, causal, scale)
    np.testing.assert_allclose(dv[0, 0, :, 0], [_frac(x) for x in exp["dv"]], atol=1e-14)
    np.testing.assert_allclose(dq[0, 0, :, 0], [_frac(x) * scale for x in exp["dq_over_ln2"]],
                               atol=1e-14)
    np.testing.assert_allclose(dk[0, 0, :, 0], [_frac(x) * scale for x in exp["dk_over_ln2"]],
                               atol=1e-14)


# ------------------------------------------------------------------ brute force
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("d", [1, 2, 4, 8])
def test_matches_scalar_brute_force(causal, n, d):
    r = _rng(100 + 7 * n + d)
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    v = np.concatenate([v, r.standard_normal((n, 3))], axis=1)  # d_v != d_k
    scale = 1.0 / math.sqrt(d)
    o, lse = ora.head_fwd(q, k, v, causal, scale)
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-13)


def test_rectangular_keys_brute_force():
    # More keys than queries, non-causal: catches a transposed operand.
    r = _rng(5)
    q, k, v = r.standard_normal((3, 4)), r.standard_normal((7, 4)), r.standard_normal((7, 2))
    o, lse = ora.head_fwd(q, k, v, False, 0.37)
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), False, 0.37)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-13)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-13)


# ----------------------------------------------------------------- closed forms
def test_single_key_gives_v_and_logit():
    r = _rng(1)
    q, k, v = r.standard_normal((1, 8)), r.standard_normal((1, 8)), r.standard_normal((1, 8))
    for causal in (False, True):
        o, lse = ora.head_fwd(q, k, v, causal, 0.3)
        np.testing.assert_allclose(o, v, atol=1e-15)
        np.testing.assert_allclose(lse, [0.3 * float(q[0] @ k[0])], atol=1e-14)


def test_zero_queries_give_means():
    r = _rng(2)
    n = 12
    q = np.zeros((n, 4))
    k, v = r.standard_normal((n, 4)), r.standard_normal((n, 5))
    o, lse = ora.head_fwd(q, k, v, False, 0.5)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, np.full(n, math.log(n)), atol=1e-14)
    o, lse = ora.head_fwd(q, k, v, True, 0.5)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, prefix, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), atol=1e-14)


def test_causal_first_row_is_first_value():
    r = _rng(3)
    q, k, v = (r.standard_normal((9, 6)) for _ in range(3))
    o, _ = ora.head_fwd(q, k, v, True, 0.4)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)


def test_dominant_key_selects_its_value():
    r = _rng(4)
    n, d = 10, 8
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    k[6] = 60.0 * q[2] / np.linalg.norm(q[2])   # logit for (2, 6) far above the rest
    o, _ = ora.head_fwd(q, k, v, False, 1.0)
    np.testing.assert_allclose(o[2], v[6], atol=1e-6)


# ------------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    r = _rng(6)
    q, k = r.standard_normal((33, 16)), r.standard_normal((33, 16))
    p = ora.head_probs(q, k, causal, 0.25)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(p >= 0)
    if causal:
        assert np.all(np.triu(p, 1) == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_value_invariants(causal):
    r = _rng(7)
    n, d = 40, 8
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    const = np.tile(r.standard_normal(d), (n, 1))
    o, _ = ora.head_fwd(q, k, const, causal, 0.35)
    np.testing.assert_allclose(o, const, atol=1e-13)
    o, _ = ora.head_fwd(q, k, v, causal, 0.35)
    a, b = 2.5, r.standard_normal(d)
    o2, _ = ora.head_fwd(q, k, a * v + b, causal, 0.35)
    np.testing.assert_allclose(o2, a * o + b, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_changes_only_lse(causal):
    r = _rng(8)
    n, d = 30, 8
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    u = r.standard_normal(d)
    o, lse = ora.head_fwd(q, k, v, causal, 0.3)
    o2, lse2 = ora.head_fwd(q, k + u, v, causal, 0.3)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + 0.3 * (q @ u), atol=1e-12)


def test_joint_key_permutation_noncausal():
    r = _rng(9)
    n, d = 25, 8
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    perm = r.permutation(n)
    o, lse = ora.head_fwd(q, k, v, False, 0.3)
    o2, lse2 = ora.head_fwd(q, k[perm], v[perm], False, 0.3)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)


def test_row_blocking_is_invisible(monkeypatch):
    r = _rng(10)
    q, k, v = (r.standard_normal((50, 8)) for _ in range(3))
    o, lse = ora.head_fwd(q, k, v, True, 0.3)
    monkeypatch.setattr(ora, "ROW_BLOCK", 7)
    o2, lse2 = ora.head_fwd(q, k, v, True, 0.3)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-14)


def test_selected_rows_and_heads_match_full():
    r = _rng(11)
    q, k, v = (r.standard_normal((2, 3, 20, 8)) for _ in range(3))
    o, lse = ora.attention_fwd(q, k, v, True, 0.3)
    rows = np.array([0, 5, 19])
    heads = [(1, 2), (0, 1)]
    o2, lse2 = ora.attention_fwd(q, k, v, True, 0.3, heads=heads, rows=rows, workers=2)
    for t, (b, h) in enumerate(heads):
        np.testing.assert_allclose(o2[t], o[b, h, rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse2[t], lse[b, h, rows], rtol=0, atol=1e-14)


# ------------------------------------------------------- online softmax model
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("trial", range(6))
def test_block_split_equals_one_shot(causal, trial):
    r = _rng(200 + trial)
    n = 48
    q, k, v = (3.0 * r.standard_normal((n, 16)) for _ in range(3))
    o, lse = ora.head_fwd(q, k, v, causal, 0.25)
    if trial == 0:
        cuts = []                                  # one block
    elif trial == 1:
        cuts = list(range(1, n))                   # n blocks of one key
    else:
        cuts = sorted(r.choice(np.arange(1, n), size=int(r.integers(1, 12)), replace=False))
    o2, lse2 = ora.online_softmax_attention(q, k, v, causal, 0.25, cuts)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


# ------------------------------------------------------------------- backward
def _fd_check(causal, seed):
    r = _rng(seed)
    n, d = 9, 4
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    scale = 0.6
    dq, dk, dv = ora.head_bwd(q, k, v, do, causal, scale)

    def loss(qq, kk, vv):
        o, _ = ora.head_fwd(qq, kk, vv, causal, scale)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        idx = [(i, c) for i in range(n) for c in range(d)]
        for (i, c) in idx:
            xp, xm = x.copy(), x.copy()
            xp[i, c] += h
            xm[i, c] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(args_p["q"], args_p["k"], args_p["v"])
                  - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(fd - g[i, c]) <= 1e-6 * max(1.0, abs(g[i, c])), (name, i, c, fd, g[i, c])


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_finite_differences(causal):
    _fd_check(causal, 300 + int(causal))


def test_gradient_against_scalar_brute_force_loss():
    # Central differences of the pure-Python loss pin dQ/dK/dV independently
    # of the numpy forward as well.
    r = _rng(12)
    n, d = 5, 3
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    scale = 0.7
    dq, dk, dv = ora.head_bwd(q, k, v, do, True, scale)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for (i, c) in [(0, 0), (2, 1), (4, 2), (3, 0)]:
            xp, xm = x.copy(), x.copy()
            xp[i, c] += h
            xm[i, c] -= h
            def L(z):
                qq, kk, vv = (z if x is q else q), (z if x is k else k), (z if x is v else v)
                return brute.loss(qq.tolist(), kk.tolist(), vv.tolist(), do.tolist(), True, scale)
            fd = (L(xp) - L(xm)) / (2 * h)
            assert abs(fd - g[i, c]) <= 1e-6 * max(1.0, abs(g[i, c]))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    r = _rng(13)
    n, d = 37, 8
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = ora.head_bwd(q, k, v, do, causal, 0.3)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    u = r.standard_normal(d)
    dq2, _, _ = ora.head_bwd(q, k + u, v, do, causal, 0.3)
    np.testing.assert_allclose(dq2, dq, atol=1e-12)


def test_backward_row_blocking_is_invisible(monkeypatch):
    r = _rng(14)
    q, k, v, do = (r.standard_normal((30, 4)) for _ in range(4))
    ref = ora.head_bwd(q, k, v, do, True, 0.5)
    monkeypatch.setattr(ora, "ROW_BLOCK", 4)
    got = ora.head_bwd(q, k, v, do, True, 0.5)
    for a, b in zip(ref, got):
        np.testing.assert_allclose(a, b, atol=1e-13)


# ------------------------------------------------- library special case (torch)
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_float64_sdpa_and_autograd(causal):
    torch = pytest.importorskip("torch")
    r = _rng(15)
    B, H, N, d = 2, 2, 19, 8
    q, k, v, do = (r.standard_normal((B, H, N, d)) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.tensor(do))
    o, _ = ora.attention_fwd(q, k, v, causal, scale)
    dq, dk, dv = ora.attention_bwd(q, k, v, do, causal, scale)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


# ------------------------------------------- shared K/V heads (MQA / GQA)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3), (3, 3)])
def test_grouped_heads_against_torch_sdpa_enable_gqa(causal, H, Hkv):
    """torch's fp64 SDPA with enable_gqa (K/V heads repeated so that
    consecutive query heads share one) and its autograd, as the library
    special case for grouped heads."""
    torch = pytest.importorskip("torch")
    r = _rng(30 + H + Hkv)
    B, N, d = 2, 13, 4
    q, do = (r.standard_normal((B, H, N, d)) for _ in range(2))
    k, v = (r.standard_normal((B, Hkv, N, d)) for _ in range(2))
    scale = 0.7
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    to.backward(torch.tensor(do))
    o, _ = ora.attention_fwd(q, k, v, causal, scale)
    dq, dk, dv = ora.attention_bwd(q, k, v, do, causal, scale)
    assert dk.shape == k.shape and dv.shape == v.shape
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_gradients_match_finite_differences(causal):
    """dK, dV of a shared K/V head against central differences of the loss
    sum(O * dO) taken through the forward (which reads that head G times)."""
    r = _rng(41)
    B, H, Hkv, N, d = 1, 4, 2, 7, 3
    q, do = (r.standard_normal((B, H, N, d)) for _ in range(2))
    k, v = (r.standard_normal((B, Hkv, N, d)) for _ in range(2))
    scale, h = 0.6, 1e-6
    _, dk, dv = ora.attention_bwd(q, k, v, do, causal, scale)

    def loss(kk, vv):
        o, _ = ora.attention_fwd(q, kk, vv, causal, scale)
        return float(np.sum(o * do))

    for _ in range(24):
        idx = tuple(int(r.integers(0, n)) for n in k.shape)
        for which, grad in (("k", dk), ("v", dv)):
            kp, km, vp, vm = k.copy(), k.copy(), v.copy(), v.copy()
            if which == "k":
                kp[idx] += h
                km[idx] -= h
            else:
                vp[idx] += h
                vm[idx] -= h
            fd = (loss(kp, vp) - loss(km, vm)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def test_identical_query_heads_share_results():
    """Multi-query attention with every query head (and dO) equal: every head
    gives the single-head result, and the shared K/V head's gradient is G times
    the single-head gradient (scalar brute force for the forward)."""
    r = _rng(42)
    G, N, d = 3, 6, 2
    q1, do1 = r.standard_normal((N, d)), r.standard_normal((N, d))
    k1, v1 = r.standard_normal((N, d)), r.standard_normal((N, d))
    q = np.broadcast_to(q1, (1, G, N, d)).copy()
    do = np.broadcast_to(do1, (1, G, N, d)).copy()
    k, v = k1[None, None], v1[None, None]
    o, lse = ora.attention_fwd(q, k, v, True, 0.9)
    ob, lb = brute.attention(q1.tolist(), k1.tolist(), v1.tolist(), True, 0.9)
    for g in range(G):
        np.testing.assert_allclose(o[0, g], ob, atol=1e-13)
        np.testing.assert_allclose(lse[0, g], lb, atol=1e-13)
    _, dk, dv = ora.attention_bwd(q, k, v, do, True, 0.9)
    _, dk1, dv1 = ora.head_bwd(q1, k1, v1, do1, True, 0.9)
    np.testing.assert_allclose(dk[0, 0], G * dk1, atol=1e-12)
    np.testing.assert_allclose(dv[0, 0], G * dv1, atol=1e-12)


def test_group_mapping_is_pinned():
    """The torch pin tells the consecutive-heads mapping (h // G) apart from an
    interleaved one (h % Hkv): on the same inputs the two disagree."""
    r = _rng(43)
    q = r.standard_normal((1, 4, 5, 2))
    k, v = r.standard_normal((1, 2, 5, 2)), r.standard_normal((1, 2, 5, 2))
    o, _ = ora.attention_fwd(q, k, v, False, 1.0)
    o_interleaved = np.stack([ora.head_fwd(q[0, h], k[0, h % 2], v[0, h % 2], False, 1.0,
                                           np.arange(5))[0] for h in range(4)])
    assert not np.allclose(o[0], o_interleaved)


# ------------------------------------------------ decoding (queries at the end)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 9), (3, 9), (4, 4), (5, 37)])
def test_decode_equals_last_rows_of_square_problem(causal, Nq, Nk):
    """Decoding Nq queries against Nk keys equals the last Nq rows of the square
    problem whose last Nq query rows are those queries (earlier rows arbitrary);
    the square problem is pinned above."""
    r = _rng(50 + Nq + Nk)
    B, H, Hkv, d = 1, 4, 2, 3
    q = r.standard_normal((B, H, Nq, d))
    k, v = r.standard_normal((B, Hkv, Nk, d)), r.standard_normal((B, Hkv, Nk, d))
    full = r.standard_normal((B, H, Nk, d))
    full[:, :, Nk - Nq:] = q
    o, lse = ora.decode_fwd(q, k, v, causal, 0.8)
    fo, fl = ora.attention_fwd(full, k, v, causal, 0.8)
    np.testing.assert_allclose(o, fo[:, :, Nk - Nq:], atol=1e-13)
    np.testing.assert_allclose(lse, fl[:, :, Nk - Nq:], atol=1e-13)


def test_decode_single_query_sees_every_key():
    """One query: causal or not, it attends to all Nk keys (scalar brute force)."""
    r = _rng(56)
    q, k, v = r.standard_normal((1, 4)), r.standard_normal((11, 4)), r.standard_normal((11, 2))
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), False, 0.6)
    for causal in (False, True):
        o, lse = ora.decode_fwd(q[None, None], k[None, None], v[None, None], causal, 0.6)
        np.testing.assert_allclose(o[0, 0], ob, atol=1e-13)
        np.testing.assert_allclose(lse[0, 0], lb, atol=1e-13)


# ----------------------------------------- rectangular score matrices (Nq != Nk)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(3, 9), (9, 3), (1, 4), (4, 1), (7, 7)])
def test_rect_against_square_problem(causal, Nq, Nk):
    """Nq <= Nk: the last Nq rows of the square problem whose last query rows
    are these. Nq > Nk: with the mask the first Nq - Nk rows see no key (O = 0,
    lse = -inf) and the rest are the square problem of size Nk; without it
    every row is the square problem's row with the same keys (brute force)."""
    r = _rng(70 + 10 * Nq + Nk)
    B, H, Hkv, d = 1, 2, 1, 3
    q = r.standard_normal((B, H, Nq, d))
    k, v = r.standard_normal((B, Hkv, Nk, d)), r.standard_normal((B, Hkv, Nk, d))
    o, lse = ora.rect_fwd(q, k, v, causal, 0.7)
    if Nq <= Nk:
        full = r.standard_normal((B, H, Nk, d))
        full[:, :, Nk - Nq:] = q
        fo, fl = ora.attention_fwd(full, k, v, causal, 0.7)
        np.testing.assert_allclose(o, fo[:, :, Nk - Nq:], atol=1e-13)
        np.testing.assert_allclose(lse, fl[:, :, Nk - Nq:], atol=1e-13)
    elif causal:
        np.testing.assert_array_equal(o[:, :, :Nq - Nk], 0.0)
        assert np.all(np.isneginf(lse[:, :, :Nq - Nk]))
        fo, fl = ora.attention_fwd(q[:, :, Nq - Nk:], k, v, True, 0.7)
        np.testing.assert_allclose(o[:, :, Nq - Nk:], fo, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, Nq - Nk:], fl, atol=1e-13)
    else:
        for h in range(H):
            ob, lb = brute.attention(q[0, h].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), False, 0.7)
            np.testing.assert_allclose(o[0, h], ob, atol=1e-13)
            np.testing.assert_allclose(lse[0, h], lb, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(3, 8), (8, 3), (1, 5), (5, 1), (6, 6)])
def test_rect_gradients_match_finite_differences(causal, Nq, Nk):
    """The rectangular backward against central differences of the
    rectangular forward's loss sum(O * dO), shared K/V head included (two
    query heads on one K/V head), every element of dQ, dK, dV."""
    r = _rng(500 + 10 * Nq + Nk + int(causal))
    B, H, Hkv, d = 1, 2, 1, 3
    q, do = r.standard_normal((B, H, Nq, d)), r.standard_normal((B, H, Nq, d))
    k, v = r.standard_normal((B, Hkv, Nk, d)), r.standard_normal((B, Hkv, Nk, d))
    scale = 0.6
    dq, dk, dv = ora.rect_bwd(q, k, v, do, causal, scale)

    def loss(qq, kk, vv):
        o, _ = ora.rect_fwd(qq, kk, vv, causal, scale)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a_p = {"q": q, "k": k, "v": v}
            a_m = dict(a_p)
            a_p[name], a_m[name] = xp, xm
            fd = (loss(a_p["q"], a_p["k"], a_p["v"]) - loss(a_m["q"], a_m["k"], a_m["v"])) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(3, 9), (1, 4), (7, 7), (2, 16)])
def test_rect_backward_against_square_problem(causal, Nq, Nk):
    """Nq <= Nk: the gradients of the square problem of size Nk whose last Nq
    query rows are these and whose other rows carry dO = 0: dK, dV equal, dQ
    equals its last Nq rows (and its other rows are 0)."""
    r = _rng(600 + 10 * Nq + Nk)
    B, H, Hkv, d = 1, 4, 2, 5
    q, do = r.standard_normal((B, H, Nq, d)), r.standard_normal((B, H, Nq, d))
    k, v = r.standard_normal((B, Hkv, Nk, d)), r.standard_normal((B, Hkv, Nk, d))
    dq, dk, dv = ora.rect_bwd(q, k, v, do, causal, 0.45)
    fq = r.standard_normal((B, H, Nk, d))
    fq[:, :, Nk - Nq:] = q
    fdo = np.zeros((B, H, Nk, d))
    fdo[:, :, Nk - Nq:] = do
    sq, sk, sv = ora.attention_bwd(fq, k, v, fdo, causal, 0.45)
    np.testing.assert_allclose(dq, sq[:, :, Nk - Nq:], atol=1e-13)
    np.testing.assert_array_equal(sq[:, :, :Nk - Nq], 0.0)
    np.testing.assert_allclose(dk, sk, atol=1e-13)
    np.testing.assert_allclose(dv, sv, atol=1e-13)


@pytest.mark.parametrize("Nq,Nk", [(5, 12), (12, 12), (1, 7)])
def test_rect_backward_against_torch_sdpa_bottom_right_mask(Nq, Nk):
    """torch fp64 scaled_dot_product_attention with an explicit boolean mask
    that keeps key j for query row i iff j <= Nk - Nq + i, and autograd."""
    torch = pytest.importorskip("torch")
    r = _rng(700 + Nq + Nk)
    B, H, d = 2, 2, 6
    q, do = r.standard_normal((B, H, Nq, d)), r.standard_normal((B, H, Nq, d))
    k, v = r.standard_normal((B, H, Nk, d)), r.standard_normal((B, H, Nk, d))
    scale = 1.0 / math.sqrt(d)
    keep = torch.tensor(np.arange(Nk)[None, :] <= (Nk - Nq + np.arange(Nq))[:, None])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep, scale=scale)
    to.backward(torch.tensor(do))
    o, _ = ora.rect_fwd(q, k, v, True, scale)
    dq, dk, dv = ora.rect_bwd(q, k, v, do, True, scale)
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_rect_backward_rows_without_keys():
    """Causal with Nq > Nk: the first Nq - Nk rows keep no key, so their dQ is
    0 and they add nothing to dK, dV; the rest is the square problem of size
    Nk."""
    r = _rng(710)
    Nq, Nk, d = 11, 4, 3
    q, do = r.standard_normal((1, 1, Nq, d)), r.standard_normal((1, 1, Nq, d))
    k, v = r.standard_normal((1, 1, Nk, d)), r.standard_normal((1, 1, Nk, d))
    dq, dk, dv = ora.rect_bwd(q, k, v, do, True, 0.8)
    np.testing.assert_array_equal(dq[:, :, :Nq - Nk], 0.0)
    sq, sk, sv = ora.attention_bwd(q[:, :, Nq - Nk:], k, v, do[:, :, Nq - Nk:], True, 0.8)
    np.testing.assert_allclose(dq[:, :, Nq - Nk:], sq, atol=1e-13)
    np.testing.assert_allclose(dk, sk, atol=1e-13)
    np.testing.assert_allclose(dv, sv, atol=1e-13)


def test_rect_pins_catch_top_left_alignment(monkeypatch):
    """A backward that aligns the mask top-left (ignores the row offset)
    fails the finite-difference pin."""
    orig = ora.head_bwd

    def head_bwd(q, k, v, do, causal, scale, pos0=0):
        return orig(q, k, v, do, causal, scale, 0)

    monkeypatch.setattr(ora, "head_bwd", head_bwd)
    with pytest.raises(AssertionError):
        test_rect_gradients_match_finite_differences(True, 3, 8)


def test_rect_dq_rows_match_full_backward():
    r = _rng(711)
    Nq, Nk, d = 9, 30, 4
    q, do = r.standard_normal((Nq, d)), r.standard_normal((Nq, d))
    k, v = r.standard_normal((Nk, d)), r.standard_normal((Nk, d))
    rows = np.array([0, 4, 8])
    for causal in (False, True):
        dq, _, _ = ora.head_bwd(q, k, v, do, causal, 0.4, pos0=Nk - Nq)
        got = ora.head_dq_rows(q, k, v, do, causal, 0.4, rows, pos0=Nk - Nq)
        np.testing.assert_allclose(got, dq[rows], rtol=0, atol=1e-13)


# ------------------------------------------------------ planted-mistake checks
def _brute_mismatch():
    r = _rng(16)
    q, k, v = r.standard_normal((6, 3)), r.standard_normal((6, 3)), r.standard_normal((6, 2))
    try:
        o, lse = ora.head_fwd(q, k, v, True, 0.8)
    except Exception:
        return True
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), True, 0.8)
    return not (np.allclose(o, ob, atol=1e-12) and np.allclose(lse, lb, atol=1e-12))


@pytest.mark.parametrize("mutation", ["no_scale", "no_mask", "mask_upper", "transpose_k",
                                      "lse_without_max"])
def test_pins_catch_planted_forward_mistakes(monkeypatch, mutation):
    orig_scores, orig_softmax = ora._scores, ora._softmax_rows

    def scores(q_rows, k, rows, causal, scale):
        if mutation == "no_scale":
            return orig_scores(q_rows, k, rows, causal, 1.0)
        if mutation == "no_mask":
            return orig_scores(q_rows, k, rows, False, scale)
        if mutation == "mask_upper":
            s = scale * (q_rows @ k.T)
            j = np.arange(k.shape[0])
            return np.where(j[None, :] < rows[:, None], -np.inf, s)
        if mutation == "transpose_k":
            return orig_scores(q_rows, k[::-1], rows, causal, scale)
        return orig_scores(q_rows, k, rows, causal, scale)

    def softmax(s):
        p, lse = orig_softmax(s)
        if mutation == "lse_without_max":
            m = np.max(s, axis=1)
            lse = lse - m
        return p, lse

    monkeypatch.setattr(ora, "_scores", scores)
    monkeypatch.setattr(ora, "_softmax_rows", softmax)
    assert _brute_mismatch()


@pytest.mark.parametrize("mutation", ["no_D", "dk_unscaled", "dv_not_transposed", "ds_sign"])
def test_pins_catch_planted_backward_mistakes(monkeypatch, mutation):
    orig = ora.head_bwd

    def head_bwd(q, k, v, do, causal, scale):
        dq, dk, dv = orig(q, k, v, do, causal, scale)
        if mutation == "no_D":
            p = ora.head_probs(q, k, causal, scale)
            ds = p * (do @ v.T)
            dq = scale * ds @ k
        elif mutation == "dk_unscaled":
            dk = dk / scale
        elif mutation == "dv_not_transposed":
            p = ora.head_probs(q, k, causal, scale)
            dv = p @ do
        elif mutation == "ds_sign":
            dq = -dq
        return dq, dk, dv

    monkeypatch.setattr(ora, "head_bwd", head_bwd)
    with pytest.raises(AssertionError):
        _fd_check(True, 301)


def test_dq_rows_match_full_backward():
    r = _rng(17)
    q, k, v, do = (r.standard_normal((40, 8)) for _ in range(4))
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        dq, _, _ = ora.head_bwd(q, k, v, do, causal, 0.4)
        np.testing.assert_allclose(ora.head_dq_rows(q, k, v, do, causal, 0.4, rows), dq[rows],
                                   rtol=0, atol=1e-13)
