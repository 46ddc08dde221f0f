"""Pure-Python scalar attention, for tiny shapes only.

TEST INFRASTRUCTURE (see ``oracle/attention.py`` for who may use ``oracle/``).

No numpy: every sum is ``math.fsum`` (exactly rounded) and every exponential
``math.exp``, straight from the definition on the "FlashAttention" page
(systems-analysis.ru), section "Problem of standard attention":
Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V, with the causal variant
keeping keys j <= i. It pins the numpy oracle: the two share no code.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

Matrix = List[List[float]]


def attention(q: Sequence[Sequence[float]], k: Sequence[Sequence[float]],
              v: Sequence[Sequence[float]], causal: bool, scale: float
              ) -> Tuple[Matrix, List[float]]:
    """Returns (O, lse) for one head given as nested lists."""
    nq, nk = len(q), len(k)
    out: Matrix = []
    lses: List[float] = []
    for i in range(nq):
        keys = [j for j in range(nk) if not (causal and j > i)]
        if not keys:
            out.append([0.0] * len(v[0]))
            lses.append(-math.inf)
            continue
        logits = [scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i])))
                  for j in keys]
        top = max(logits)
        w = [math.exp(x - top) for x in logits]
        total = math.fsum(w)
        out.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(keys)) / total
                    for c in range(len(v[0]))])
        lses.append(top + math.log(total))
    return out, lses


def loss(q, k, v, do, causal: bool, scale: float) -> float:
    """The scalar L = sum_ic O_ic * dO_ic whose gradients the backward returns."""
    o, _ = attention(q, k, v, causal, scale)
    return math.fsum(o[i][c] * do[i][c] for i in range(len(o)) for c in range(len(o[0])))
