"""fa_decode_noalloc (no allocation; the library's fixed device buffer in place
of a workspace) against fa_decode, through the C ABI: equal bits on two calls
in a row, the second smaller than the first, and a clear error for a problem
whose partial results exceed the buffer."""
import numpy as np
import pytest

from exact_attention_41_amd import workloads as wl
from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    from exact_attention_41_amd import _lib
    _lib.load()
    return fa


CASES = [(8, 32, 8, 1, 32768, 128, True, 7),     # the 32k-context decoding workload
         (2, 8, 2, 4, 1000, 64, True, 41),       # smaller, ragged, four query rows
         (1, 4, 4, 3, 517, 256, False, 42)]      # smaller again, d = 256


def _inputs(B, H, Hkv, Nq, Nk, d, seed):
    inp = wl.make_decode_inputs(B, H, Hkv, Nq, Nk, d, seed)
    return tuple(wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))


def test_noalloc_equals_fa_decode_on_consecutive_calls(fa):
    import torch
    outs = []
    for B, H, Hkv, Nq, Nk, d, causal, seed in CASES:
        say(f"fa_decode_noalloc B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} "
            f"seed={seed} workspace={fa.fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d)}")
        q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, seed)
        o_ref, l_ref = fa.fa_decode(q, k, v, causal=causal)
        o, lse = fa.fa_decode_noalloc(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32))
        outs.append((o, lse))
    # the last call's scratch contents did not disturb the earlier results
    assert all(torch.isfinite(o.float()).all() for o, _ in outs)


def test_noalloc_rejects_problems_beyond_its_buffer(fa):
    import torch
    from exact_attention_41_amd import _lib
    B, H, Hkv, Nq, Nk, d = 2047, 1, 1, 1, 64, 128
    need = fa.fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d)
    say(f"fa_decode_noalloc oversize B={B} workspace={need}")
    assert need > 40 << 20
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, Nk, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_noalloc(q, k, k, causal=True)
    assert e.value.status == 3      # FA_ERR_WORKSPACE
