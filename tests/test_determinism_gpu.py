"""Repeated calls give identical bits (the "FlashAttention-2" page,
systems-analysis.info, section "Performance", calls the method exact and
deterministic): every output element has one writer and a fixed order of
accumulation, in the forward, the backward (no floating-point atomics),
decoding (the merge walks the key ranges in order) and the fp8 forward. Run
at the benchmark sizes, with other work on the device between the calls."""
import pytest

from exact_attention_41_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import exact_attention_41_amd as fa
    from exact_attention_41_amd import _lib
    _lib.load()
    return fa


def _same(runs):
    import torch
    torch.cuda.synchronize()
    first = runs[0]
    for other in runs[1:]:
        for a, b in zip(first, other):
            assert torch.equal(a, b)


def _noise():
    import torch
    x = torch.randn(1 << 22, device="cuda")
    return (x * 2).sum()


def test_forward_and_backward_are_deterministic(fa):
    w = wl.WORKLOADS["bf16_b4h16n4096d128_causal_bwd"]
    print(f"determinism fwd+bwd {w.name}", flush=True)
    inp = wl.workload_inputs(w)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    fwd, bwd = [], []
    for _ in range(3):
        o, lse = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
        fwd.append((o, lse))
        bwd.append(fa.fa_bwd(q, k, v, o, do, lse, causal=True, scale=w.scale))
        _noise()
    _same(fwd)
    _same(bwd)


def test_wide_fp8_and_decode_are_deterministic(fa):
    w = wl.WIDE_WORKLOADS["bf16_b4h8n4096d256_causal"]
    print(f"determinism d=256 {w.name}", flush=True)
    inp = wl.make_inputs(w.B, w.H, w.N, w.d, "bf16", w.seed, with_do=True)
    q, k, v, do = (wl.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v, inp.do))
    runs = []
    for _ in range(2):
        o, lse = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
        runs.append((o, lse) + tuple(fa.fa_bwd(q, k, v, o, do, lse, causal=True, scale=w.scale)))
        _noise()
    _same(runs)
    del q, k, v, do, runs

    f8 = wl.FP8_WORKLOADS["fp8_b4h16n4096d128_causal"]
    print(f"determinism fp8 {f8.name}", flush=True)
    inp8 = wl.make_fp8_inputs(f8.B, f8.H, f8.H, f8.N, f8.N, f8.d, f8.seed)
    q8, k8, v8 = (wl.fp8_to_device(x) for x in (inp8.q8, inp8.k8, inp8.v8))
    runs = []
    for _ in range(2):
        runs.append(fa.fa_fwd_fp8(q8, k8, v8, inp8.dq, inp8.dk, inp8.dv, causal=True,
                                  scale=f8.scale))
        _noise()
    _same(runs)
    del q8, k8, v8, runs

    dw = wl.DECODE_WORKLOADS["bf16_decode_b8h32kv8q1k32768d128"]
    print(f"determinism decode {dw.name}", flush=True)
    dinp = wl.make_decode_inputs(dw.B, dw.H, dw.Hkv, dw.Nq, dw.Nk, dw.d, dw.seed)
    q, k, v = (wl.to_device(x, "bf16") for x in (dinp.q, dinp.k, dinp.v))
    runs = []
    for _ in range(2):
        runs.append(fa.fa_decode(q, k, v, causal=dw.causal, scale=dw.scale))
        _noise()
    _same(runs)
