"""fa_attention (torch autograd over fa_fwd_rect / fa_bwd_rect, with O's
rounding residual passed from the one to the other): the output and the
gradients torch computes through it are the entry points' own bits, and they
match the fp64 oracle."""
import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from oracle import attention as ora
from parity_util import check_bf16, say, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_autograd_matches_entry_points_and_oracle(causal):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 150, 260, 128
    say(f"fa_attention autograd B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} seed=96")
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, d, seed=96, with_do=True)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fa.fa_attention(qa, ka, va, causal=causal)
    (o.float() * do.float()).sum().backward()
    # fa_attention keeps O's rounding residual in the forward and hands it to the backward
    o_res = torch.empty_like(q)
    o2, lse2 = fa.fa_fwd_rect(q, k, v, causal=causal, o_res=o_res)
    g2 = fa.fa_bwd_rect(q, k, v, o2, do, lse2, causal=causal, o_res=o_res)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for a, b in zip((qa.grad, ka.grad, va.grad), g2):
        assert torch.equal(a, b)
    scale = float(np.float32(1 / np.sqrt(d)))
    q64, k64, v64, do64 = inp.as_float64()
    rq, rk, rv = ora.rect_bwd(q64, k64, v64, do64, causal, scale, workers=None)
    check_bf16("dQ", to_np(qa.grad), rq)
    check_bf16("dK", to_np(ka.grad), rk)
    check_bf16("dV", to_np(va.grad), rv)
