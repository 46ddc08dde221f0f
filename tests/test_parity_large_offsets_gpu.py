"""Forward and backward on tensors of more than 2^31 elements (4.3 GB each in
bf16): B=1, H=4104, N=4096, d=128, causal, in the launch configuration of any
other call. Every element offset past 2^31 must be formed in 64 bits; the
first, a middle and the last head (whose elements all lie past 2^31) are
compared with the fp64 oracle on every element. About 47 GB of device memory.

The inputs are drawn on the device (workloads.device_normal_bf16); the heads
given to the oracle are copied back from the device.
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


def test_forward_backward_past_2_31_elements(fa):
    import torch
    B, H, N, d, causal = 1, 4104, 4096, 128, True
    assert B * H * N * d > 2 ** 31
    scale = float(np.float32(1 / np.sqrt(d)))
    say(f"fa_fwd/fa_bwd B={B} H={H} N={N} d={d} causal={causal} seeds 51-54 "
        f"({B * H * N * d} elements per tensor)")
    # the device generator: the same seed gives the same bits on the GPU too
    a, b = (wl.device_normal_bf16((3, 1000), 51) for _ in range(2))
    assert a.is_cuda and torch.equal(a.view(torch.int16), b.view(torch.int16))
    q, k, v, do = (wl.device_normal_bf16((B, H, N, d), seed) for seed in (51, 52, 53, 54))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for h in (0, H // 2, H - 1):
        say(f"  head {h}")
        q64, k64, v64, do64 = (to_np(x[:, h:h + 1]) for x in (q, k, v, do))
        ro, rl = ora.attention_fwd(q64, k64, v64, causal, scale, workers=None)
        rq, rk, rv = ora.attention_bwd(q64, k64, v64, do64, causal, scale, workers=None)
        check_bf16(f"O[{h}]", to_np(o[:, h:h + 1]), ro)
        check_abs(f"lse[{h}]", to_np(lse[:, h:h + 1]), rl, LSE_ATOL)
        check_bf16(f"dQ[{h}]", to_np(dq[:, h:h + 1]), rq)
        check_bf16(f"dK[{h}]", to_np(dk[:, h:h + 1]), rk)
        check_bf16(f"dV[{h}]", to_np(dv[:, h:h + 1]), rv)
