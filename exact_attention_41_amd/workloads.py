"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage type.
It holds none of the attention arithmetic, so that both the fp64 oracle (test
infrastructure) and the HIP path can be fed from it without sharing any of the
method's code.

Recipe (the same for every workload):
  * generator ``numpy.random.Generator(PCG64(seed))``;
  * ``standard_normal(dtype=float32)`` draws, tensor by tensor in the order
    q, k, v, then dO, each of shape [B, H, N, d] (row-major; k and v have
    [B, Hkv, N, d] when Hkv K/V heads are shared by the H query heads);
  * an optional fp32 multiplier on q and k (the sharpened-softmax workload);
  * one round-to-nearest-even cast to bfloat16 (except fp32 workloads);
  * fp8 workloads instead divide each tensor by its own factor
    fp32(max|x| / 448) and cast it to OCP e4m3 (round to nearest even); the
    real inputs are factor * e4m3 value.

The attention problem is the scaled dot-product attention of the
"FlashAttention" page (systems-analysis.ru), section "Problem of standard
attention": O = softmax(Q K^T / sqrt(d_k)) V, per batch entry and head.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "bf16" or "f32": storage and MFMA operand type
    causal: bool
    seed: int
    qk_mult: float = 1.0
    backward: bool = False
    description: str = ""
    Hkv: Optional[int] = None      # K/V heads (None: H, ordinary multi-head)

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32, the value passed through the C ABI."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def fwd_flops(self) -> float:
        """Counted forward flops: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def bwd_flops(self) -> float:
        """Counted backward flops: 2.5x the forward count (five N^2*d GEMMs)."""
        return 2.5 * self.fwd_flops()


# The five synthetic workloads: sizes, value distributions and masks.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("fp32_b1h1n256d64", 1, 1, 256, 64, "f32", False, 1,
                 description="non-causal fp32 forward, B=1 H=1 N=256 d=64"),
        Workload("bf16_b8h16n2048d64", 8, 16, 2048, 64, "bf16", False, 2,
                 description="non-causal bf16 forward, B=8 H=16 N=2048 d=64"),
        Workload("bf16_b8h16n2048d64_causal", 8, 16, 2048, 64, "bf16", True, 2,
                 description="causal bf16 forward, same tensors as the non-causal case"),
        Workload("bf16_b2h32n8192d128_causal_x3", 2, 32, 8192, 128, "bf16", True, 3,
                 qk_mult=3.0,
                 description="causal bf16 forward, q and k scaled by 3 (sharp softmax)"),
        Workload("bf16_b1h16n16384d128_causal", 1, 16, 16384, 128, "bf16", True, 4,
                 description="long-sequence causal bf16 forward, O(N) extra memory"),
        Workload("bf16_b4h16n4096d128_causal_bwd", 4, 16, 4096, 128, "bf16", True, 5,
                 backward=True,
                 description="causal bf16 forward + backward with upstream dO"),
    ]
}

# Shared K/V heads: 32 query heads over 8 K/V heads (groups of 4).
GQA_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("bf16_b2h32kv8n4096d128_causal_gqa", 2, 32, 4096, 128, "bf16", True, 6,
                 backward=True, Hkv=8,
                 description="causal bf16 forward + backward, 32 query heads sharing 8 K/V heads"),
    ]
}


# Head size 256 (the largest the "FlashAttention" page, section
# "FlashAttention-2 (2023)", names): 16384 tokens per batch (a batch size
# chosen here; the pages give no benchmark shape), 8 heads of 256 =
# 2048 model width; both masks on the same tensors.
WIDE_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("bf16_b4h8n4096d256", 4, 8, 4096, 256, "bf16", False, 9,
                 description="non-causal bf16 forward, head size 256"),
        Workload("bf16_b4h8n4096d256_causal", 4, 8, 4096, 256, "bf16", True, 9,
                 description="causal bf16 forward, head size 256, same tensors"),
    ]
}


# 8-bit floating-point forward (e4m3 q, k, v with one factor per tensor):
# the headline shape, both masks on the same tensors, and a long sequence.
FP8_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("fp8_b4h16n4096d128", 4, 16, 4096, 128, "fp8", False, 11,
                 description="non-causal fp8 forward, e4m3 q, k, v, per-tensor factors"),
        Workload("fp8_b4h16n4096d128_causal", 4, 16, 4096, 128, "fp8", True, 11,
                 description="causal fp8 forward, same tensors"),
        Workload("fp8_b1h16n16384d128_causal", 1, 16, 16384, 128, "fp8", True, 12,
                 description="long-sequence causal fp8 forward"),
    ]
}


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Decoding: Nq query rows per head (the last Nq positions) against Nk keys,
    K/V shared by groups of H / Hkv query heads."""
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    description: str = ""

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def kv_bytes(self) -> int:
        """bf16 K and V, read once: the bulk of the algorithmic traffic."""
        return 2 * self.B * self.Hkv * self.Nk * self.d * 2

    def io_bytes(self) -> int:
        """All algorithmic bytes: K, V, q and O (bf16), lse (fp32)."""
        rows = self.B * self.H * self.Nq
        return self.kv_bytes() + 2 * rows * self.d * 2 + rows * 4


# A decoding step at a 32k-token context: 32 query heads over 8 K/V heads.
DECODE_WORKLOADS: Dict[str, DecodeWorkload] = {
    w.name: w
    for w in [
        DecodeWorkload("bf16_decode_b8h32kv8q1k32768d128", 8, 32, 8, 1, 32768, 128, False, 7,
                       "one new token per sequence, 8 sequences of 32768 cached keys"),
        DecodeWorkload("bf16_decode_b8h16kv4q1k32768d256", 8, 16, 4, 1, 32768, 256, False, 10,
                       "head size 256: 16 query heads over 4 K/V heads, 32768 cached keys"),
    ]
}


# A chunk of new queries against a longer cached key sequence (chunked prefill).
RECT_WORKLOADS: Dict[str, DecodeWorkload] = {
    w.name: w
    for w in [
        DecodeWorkload("bf16_prefill_b1h32kv8q4096k16384d128_causal", 1, 32, 8, 4096, 16384, 128,
                       True, 8, "4096 new tokens after 12288 cached ones, bottom-right causal"),
    ]
}


def rect_flops(w: DecodeWorkload) -> float:
    """Counted forward flops: 4*d per unmasked score element (query row i at
    position Nk - Nq + i keeps min(Nk, Nk - Nq + i + 1) keys when causal)."""
    off = w.Nk - w.Nq
    if w.causal:
        i = np.arange(w.Nq, dtype=np.float64)
        elems = float(np.clip(off + i + 1, 0, w.Nk).sum())
    else:
        elems = float(w.Nq) * w.Nk
    return 4.0 * w.d * w.B * w.H * elems


def make_decode_inputs(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int,
                       with_do: bool = False) -> Inputs:
    """Decoding (and rectangular) inputs: q [B,H,Nq,d], then k and v
    [B,Hkv,Nk,d] (then dO [B,H,Nq,d]), drawn in that order with the recipe of
    the module docstring and rounded to bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    do = bf16_round(rng.standard_normal((B, H, Nq, d), dtype=np.float32)) if with_do else None
    return Inputs(bf16_round(q), bf16_round(k), bf16_round(v), do, "bf16")


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns a float32 array whose values are exactly representable in bf16.
    NaN/Inf are not expected in these inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x_rounded: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-representable float32 values (the bf16 storage)."""
    u = np.ascontiguousarray(x_rounded, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


@dataclasses.dataclass
class Inputs:
    """Quantised inputs as float32 arrays (values exact in the storage type)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    dtype: str

    def as_float64(self):
        out = [self.q.astype(np.float64), self.k.astype(np.float64),
               self.v.astype(np.float64)]
        out.append(None if self.do is None else self.do.astype(np.float64))
        return tuple(out)


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int,
                qk_mult: float = 1.0, with_do: bool = False,
                Hkv: Optional[int] = None, v_mean: float = 0.0) -> Inputs:
    """Draw q, k, v (and dO) following the recipe in the module docstring;
    ``v_mean`` (stress inputs only) is added to v in fp32 before rounding."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    kv_shape = (B, H if Hkv is None else Hkv, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(kv_shape, dtype=np.float32)
    v = rng.standard_normal(kv_shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32) if with_do else None
    if qk_mult != 1.0:
        q = q * np.float32(qk_mult)
        k = k * np.float32(qk_mult)
    if v_mean != 0.0:
        v = v + np.float32(v_mean)
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
        if do is not None:
            do = bf16_round(do)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return Inputs(q, k, v, do, dtype)


def workload_inputs(w: Workload) -> Inputs:
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_mult,
                       with_do=w.backward, Hkv=w.Hkv)


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    """Copy a quantised float32 array to a torch tensor of the storage type."""
    import torch
    if dtype == "bf16":
        bits = bf16_bits(x).view(np.int16)
        t = torch.from_numpy(bits).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


def device_normal_bf16(shape, seed: int, device="cuda"):
    """Seeded N(0, 1) draws made on the device by torch's generator for that
    device (seeded with ``seed``), rounded once to bfloat16: for tensors too
    large to draw on the host. Whatever the oracle is given of them is copied
    back from the device, so both sides see the same values."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


# ---------------------------------------------------------------- fp8 inputs
E4M3_MAX = 448.0     # largest finite OCP e4m3 value


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 values with |x| <= 448 -> OCP e4m3 bytes, round to nearest even
    (torch's float8_e4m3fn cast on the CPU)."""
    import torch
    x = np.asarray(x, dtype=np.float32)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: values beyond 448")
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """OCP e4m3 bytes -> exact values as float64 (NaN for the two NaN codes)."""
    import torch
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8))
    return torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@dataclasses.dataclass
class Fp8Inputs:
    """e4m3 bytes of q, k, v and their dequantisation factors (fp32): the
    real inputs are descale * e4m3 value."""
    q8: np.ndarray
    k8: np.ndarray
    v8: np.ndarray
    dq: float
    dk: float
    dv: float

    def as_float64(self):
        """The real (dequantised) inputs, exact in float64."""
        return (e4m3_decode(self.q8) * self.dq, e4m3_decode(self.k8) * self.dk,
                e4m3_decode(self.v8) * self.dv)


def quantize_e4m3(x: np.ndarray) -> Tuple[np.ndarray, float]:
    """Per-tensor factor s = fp32(max|x| / 448) and the bytes of e4m3(x / s)."""
    amax = float(np.max(np.abs(x)))
    s = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    y = np.clip(x.astype(np.float32) / np.float32(s), -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(y), s


def make_fp8_inputs(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int,
                    qk_mult: float = 1.0) -> Fp8Inputs:
    """q [B,H,Nq,d], then k and v [B,Hkv,Nk,d], drawn as standard normals in
    that order (recipe of the module docstring; q and k multiplied by qk_mult)
    and quantised per tensor with quantize_e4m3."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, Nq, d), dtype=np.float32) * np.float32(qk_mult)
    k = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32) * np.float32(qk_mult)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    (q8, dq), (k8, dk), (v8, dv) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    return Fp8Inputs(q8, k8, v8, dq, dk, dv)


def fp8_to_device(b: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(b)).to(device).view(torch.float8_e4m3fn)
