"""Parity of split-K/V decoding (fa_decode) against the fp64 oracle, through
the C ABI: Nq query rows per head at the last Nq positions of Nk keys, K/V
heads shared by groups of query heads, bottom-right causal or no mask.

Every output element is compared, on small shapes (ragged key counts, one to
four queries, groups of 1 to 32, both d) and on the 32k-key decoding workload
the benchmark times.
"""
import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import LSE_ATOL, check_abs, check_bf16, say, to_np

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
    o, lse = fa.fa_decode(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


SMALL = [(1, 1, 1, 1, 1, 64), (2, 4, 1, 1, 1000, 128), (1, 8, 2, 4, 777, 128),
         (2, 32, 8, 1, 5000, 128), (1, 4, 4, 3, 64, 64), (1, 16, 2, 2, 300, 64),
         (1, 32, 1, 1, 2049, 128), (3, 2, 2, 16, 16, 128)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d", SMALL)
def test_decode_small(fa, B, H, Hkv, Nq, Nk, d, causal):
    say(f"fa_decode B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} seed=61")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, d, seed=61)
    scale = float(np.float32(1 / np.sqrt(d)))
    o, lse = _run(fa, inp, causal, scale)
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.decode_fwd(q64, k64, v64, causal, scale, workers=None)
    check_bf16("O", o, ro)
    check_abs("lse", lse, rl, LSE_ATOL)


def test_decode_workload(fa):
    w = wl.DECODE_WORKLOADS["bf16_decode_b8h32kv8q1k32768d128"]
    say(f"decode workload {w.name}: B={w.B} H={w.H} Hkv={w.Hkv} Nq={w.Nq} Nk={w.Nk} d={w.d}")
    inp = wl.make_decode_inputs(w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, w.seed)
    o, lse = _run(fa, inp, w.causal, w.scale)
    q64, k64, v64, _ = inp.as_float64()
    ro, rl = ora.decode_fwd(q64, k64, v64, w.causal, w.scale, workers=None)
    check_bf16("O (every row)", o, ro)
    check_abs("lse (every row)", lse, rl, LSE_ATOL)
