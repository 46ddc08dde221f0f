"""Parity of the rectangular forward (fa_fwd_rect: Nq query rows against Nk
keys, query row i at position Nk - Nq + i, bottom-right causal) against the
fp64 oracle, through the C ABI.

Small shapes (Nq < Nk, Nq > Nk with rows that see no key, ragged tiles,
shared K/V heads, both d) are compared on every element; the chunked-prefill
workload the benchmark times is compared on sampled rows of every head.
"""
import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import LSE_ATOL, check_abs, check_bf16, sample_rows, say, to_np

pytestmark = pytest.mark.gpu


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
    q, k, v = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o, lse = fa.fa_fwd_rect(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


SMALL = [(1, 2, 1, 100, 300, 128), (2, 4, 2, 300, 100, 64), (1, 2, 2, 64, 4096, 128),
         (1, 1, 1, 1, 1000, 128), (1, 2, 1, 513, 1025, 64), (1, 3, 3, 700, 333, 128),
         (2, 2, 1, 257, 257, 128)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d", SMALL)
def test_rect_forward_small(fa, B, H, Hkv, Nq, Nk, d, causal):
    say(f"fa_fwd_rect B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} seed=81")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, d, seed=81)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(fa, inp, causal, scale)
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.rect_fwd(q64, k64, v64, causal, scale, workers=None)
    check_bf16("O", o, ro)
    check_abs("lse", lse, rl, LSE_ATOL)


def test_rect_prefill_workload(fa):
    """4096 new queries after 12288 cached keys: sampled rows of every head."""
    import concurrent.futures as cf
    w = wl.RECT_WORKLOADS["bf16_prefill_b1h32kv8q4096k16384d128_causal"]
    G = w.H // w.Hkv
    say(f"rect workload {w.name}: B={w.B} H={w.H} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d}")
    inp = wl.make_decode_inputs(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed)
    o, lse = _run(fa, inp, w.causal, w.scale)
    q64, k64, v64, _ = inp.as_float64()
    rows = sample_rows(w.Nq, 32, seed=w.seed)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        return ora.head_fwd(q64[b, h], k64[b, h // G], v64[b, h // G], w.causal, w.scale, rows,
                            pos0=w.Nk - w.Nq)

    with cf.ThreadPoolExecutor(8) as ex:
        res = list(ex.map(one, pairs))
    ro = np.stack([r[0] for r in res])
    rl = np.stack([r[1] for r in res])
    check_bf16("O (sampled rows, all heads)", o.reshape(w.B * w.H, w.Nq, w.d)[:, rows], ro)
    check_abs("lse (sampled rows, all heads)", lse.reshape(w.B * w.H, w.Nq)[:, rows], rl, LSE_ATOL)
