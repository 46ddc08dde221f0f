"""MI355X (gfx950) fused exact attention: thin Python binding of libfa.so.

The functions below carry the names of the C entry points in include/fa.h and
only marshal torch tensors (device memory and the current stream) into those
calls; every step of the computation runs in the HIP kernels of libfa.so.
If the library is not built, every call raises: there is no fallback.

    o, lse = fa_fwd(q, k, v, causal=True)                  # bf16 [B,H,N,d]
    o, lse = fa_fwd(q, k, v, causal=True, o_res=r)         # fa_fwd_train: also O's residual
    o, lse = fa_fwd_f32(q, k, v, causal=False)             # fp32 [B,H,N,d]
    dq, dk, dv = fa_bwd(q, k, v, o, do, lse, causal=True)  # bf16
    dq, dk, dv = fa_bwd(q, k, v, o, do, lse, causal=True, o_res=r)   # fa_bwd_train
    o, lse = fa_fwd_gqa(q, k, v, causal=True)              # k, v: [B,Hkv,N,d]
    dq, dk, dv = fa_bwd_gqa(q, k, v, o, do, lse, causal=True)
    o, lse = fa_decode(q, k, v)          # q [B,H,Nq,d], k, v [B,Hkv,Nk,d]
    o, lse = fa_fwd_rect(q, k, v, causal=True)   # any Nq, Nk; bottom-right causal
    dq, dk, dv = fa_bwd_rect(q, k, v, o, do, lse, causal=True)
    o, lse = fa_fwd_fp8(q8, k8, v8, dq, dk, dv)  # e4m3 inputs with per-tensor factors
    o = fa_attention(q, k, v, causal=True)       # autograd: backward through fa_bwd_rect
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

from . import _lib

__all__ = ["fa_fwd", "fa_fwd_f32", "fa_bwd", "fa_bwd_workspace_size", "fa_status_str",
           "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq", "fa_fwd_gqa", "fa_bwd_gqa",
           "fa_bwd_gqa_workspace_size", "fa_decode", "fa_decode_workspace_size", "fa_fwd_rect",
           "fa_fwd_fp8", "fa_bwd_rect", "fa_bwd_rect_workspace_size", "fa_clock_probe",
           "fa_attention", "fa_decode_noalloc", "fa_fwd_train", "fa_bwd_train", "FAError",
           "library_path"]


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {fa_status_str(status)}")


def library_path() -> str:
    return _lib.LIB_PATH


def fa_status_str(status: int) -> str:
    return _lib.load().fa_status_str(int(status)).decode()


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().fa_bwd_workspace_size(B, H, N, d))


def fa_bwd_gqa_workspace_size(B: int, H: int, Hkv: int, N: int, d: int) -> int:
    return int(_lib.load().fa_bwd_gqa_workspace_size(B, H, Hkv, N, d))


def fa_bwd_rect_workspace_size(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(_lib.load().fa_bwd_rect_workspace_size(B, H, Hkv, Nq, Nk, d))


def _torch():
    import torch
    return torch


def _check(t, name, dtype, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_workspace(ws, device) -> int:
    """A caller's workspace: a contiguous tensor on ``device``; returns its bytes."""
    torch = _torch()
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.numel() * ws.element_size()


def _stream_ptr(device):
    return _torch().cuda.current_stream(device).cuda_stream


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _kv_heads(q, k, grouped):
    """Hkv from k's shape: equal to H unless ``grouped`` (then dividing H)."""
    if k.dim() != 4:
        raise ValueError("k must be [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1] if grouped else H
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"k has {k.shape[1]} heads, which does not divide H = {H}")
    return Hkv


def _o_res_ptr(o_res, q):
    """Device pointer of an optional o_res tensor (bf16, q's shape), or None."""
    if o_res is None:
        return None
    _check(o_res, "o_res", _torch().bfloat16, q.shape, q.device)
    return o_res.data_ptr()


def _fwd(entry, dtype, q, k, v, causal, scale, out, lse, grouped=False, o_res=None):
    torch = _torch()
    _check(q, "q", dtype)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(q, k, grouped)
    kv_shape = (B, Hkv, N, d)
    _check(k, "k", dtype, kv_shape, q.device)
    _check(v, "v", dtype, kv_shape, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(out, "out", dtype, q.shape, q.device)
    _check(lse, "lse", torch.float32, (B, H, N), q.device)
    if o_res is not None:
        # the training forward: fa_fwd_train with Nq = Nk = N
        entry = "fa_fwd_train"
        with torch.cuda.device(q.device):
            st = _lib.load().fa_fwd_train(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), _o_res_ptr(o_res, q), lse.data_ptr(),
                                          B, H, Hkv, N, N, d, int(bool(causal)),
                                          _scale(scale, d), _stream_ptr(q.device))
        if st != _lib.FA_OK:
            raise FAError(st, entry)
        return out, lse
    fn = getattr(_lib.load(), entry)
    heads = (B, H, Hkv) if grouped else (B, H)
    with torch.cuda.device(q.device):
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                *heads, N, d, int(bool(causal)), _scale(scale, d), _stream_ptr(q.device))
    if st != _lib.FA_OK:
        raise FAError(st, entry)
    return out, lse


def fa_fwd(q, k, v, causal: bool = False, scale: Optional[float] = None,
           out=None, lse=None, o_res=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """bf16 forward: returns (O, logsumexp). Calls fa_fwd of libfa.so, or, when
    ``o_res`` (a bf16 tensor of q's shape) is given, fa_fwd_train, which also
    stores O's rounding residual there for the backward."""
    return _fwd("fa_fwd", _torch().bfloat16, q, k, v, causal, scale, out, lse, o_res=o_res)


def fa_fwd_gqa(q, k, v, causal: bool = False, scale: Optional[float] = None,
               out=None, lse=None, o_res=None):
    """bf16 forward with shared K/V heads: q [B,H,N,d], k and v [B,Hkv,N,d]
    (Hkv dividing H; query head h uses K/V head h // (H // Hkv)). Returns
    (O, logsumexp); ``o_res`` as for fa_fwd. Calls fa_fwd_gqa of libfa.so."""
    return _fwd("fa_fwd_gqa", _torch().bfloat16, q, k, v, causal, scale, out, lse, grouped=True,
                o_res=o_res)


def fa_fwd_f32(q, k, v, causal: bool = False, scale: Optional[float] = None,
               out=None, lse=None):
    """fp32 forward: returns (O, logsumexp). Calls fa_fwd_f32 of libfa.so."""
    return _fwd("fa_fwd_f32", _torch().float32, q, k, v, causal, scale, out, lse)


def _bwd(entry, q, k, v, o, do, lse, causal, scale, dq, dk, dv, workspace, grouped,
         rect=False, o_res=None):
    torch = _torch()
    bf = torch.bfloat16
    _check(q, "q", bf)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    if rect:
        if not isinstance(k, torch.Tensor) or k.dim() != 4:
            raise ValueError("k must be [B, Hkv, Nk, d]")
        Hkv, Nk = k.shape[1], k.shape[2]
    else:
        Hkv, Nk = _kv_heads(q, k, grouped), N
    kv_shape = (B, Hkv, Nk, d)
    for t, n, shp in ((k, "k", kv_shape), (v, "v", kv_shape), (o, "o", q.shape),
                      (do, "do", q.shape)):
        _check(t, n, bf, shp, q.device)
    _check(lse, "lse", torch.float32, (B, H, N), q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n, shp in ((dq, "dq", q.shape), (dk, "dk", kv_shape), (dv, "dv", kv_shape)):
        _check(t, n, bf, shp, q.device)
    need = fa_bwd_rect_workspace_size(B, H, Hkv, N, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q.device)
    heads = (B, H, Hkv) if grouped or rect else (B, H)
    sizes = (N, Nk) if rect else (N,)
    res = ()
    if o_res is not None:
        # the training backward: fa_bwd_train (general heads and lengths)
        entry, heads, sizes, res = "fa_bwd_train", (B, H, Hkv), (N, Nk), (_o_res_ptr(o_res, q),)
    fn = getattr(_lib.load(), entry)
    with torch.cuda.device(q.device):
        st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), *res,
                do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                workspace.data_ptr(), ws_bytes, *heads, *sizes, d, int(bool(causal)),
                _scale(scale, d), _stream_ptr(q.device))
    if st != _lib.FA_OK:
        raise FAError(st, entry)
    return dq, dk, dv


def fa_bwd(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
           dq=None, dk=None, dv=None, workspace=None, o_res=None):
    """bf16 backward: returns (dQ, dK, dV). Calls fa_bwd of libfa.so.

    ``workspace`` may be a uint8 device tensor of at least
    fa_bwd_workspace_size(B, H, N, d) bytes; one is allocated otherwise.
    ``o_res``: the forward's rounding residual of O, if it kept one; then this
    calls fa_bwd_train (D from O in the preprocess, a cheaper dQ pass).
    """
    return _bwd("fa_bwd", q, k, v, o, do, lse, causal, scale, dq, dk, dv, workspace, False,
                o_res=o_res)


def fa_bwd_gqa(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
               dq=None, dk=None, dv=None, workspace=None, o_res=None):
    """bf16 backward of fa_fwd_gqa: returns (dQ [B,H,N,d], dK and dV [B,Hkv,N,d],
    each K/V head's gradient summed over the query heads that share it).
    Calls fa_bwd_gqa of libfa.so; ``workspace`` as for fa_bwd, of
    fa_bwd_gqa_workspace_size(B, H, Hkv, N, d) bytes."""
    return _bwd("fa_bwd_gqa", q, k, v, o, do, lse, causal, scale, dq, dk, dv, workspace, True,
                o_res=o_res)


def fa_bwd_rect(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
                dq=None, dk=None, dv=None, workspace=None, o_res=None):
    """bf16 backward of fa_fwd_rect: q, o, do [B,H,Nq,d], lse [B,H,Nq], k and v
    [B,Hkv,Nk,d]; returns (dQ [B,H,Nq,d], dK and dV [B,Hkv,Nk,d]). Query row i
    sits at position Nk - Nq + i (bottom-right causal alignment). Calls
    fa_bwd_rect of libfa.so; ``workspace`` as for fa_bwd, of
    fa_bwd_rect_workspace_size(B, H, Hkv, Nq, Nk, d) bytes."""
    return _bwd("fa_bwd_rect", q, k, v, o, do, lse, causal, scale, dq, dk, dv, workspace, True,
                rect=True, o_res=o_res)


def _bwd_common(ref, tensors, lse, workspace):
    torch = _torch()
    bf = torch.bfloat16
    _check(ref, "k", bf)
    if ref.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    B, H, N, d = ref.shape
    for t, n in tensors:
        _check(t, n, bf, ref.shape, ref.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, N), ref.device)
    if workspace is None:
        raise ValueError("workspace is required (a uint8 device tensor of "
                         "fa_bwd_workspace_size(B, H, N, d) bytes)")
    return B, H, N, d, _check_workspace(workspace, ref.device)


def fa_bwd_preprocess(q, k, v, o, do, workspace, o_res=None):
    """Phase 1 of fa_bwd: per-head scale factors, rowsum(dO * O) (O = o, or
    o + o_res when ``o_res`` is given) and the scaled fp16 transposed copies of
    q, dO and k into ``workspace``."""
    torch = _torch()
    B, H, N, d, ws = _bwd_common(k, [(q, "q"), (v, "v"), (o, "o"), (do, "do")], None, workspace)
    with torch.cuda.device(k.device):
        st = _lib.load().fa_bwd_preprocess(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           o.data_ptr(), _o_res_ptr(o_res, q), do.data_ptr(),
                                           workspace.data_ptr(), ws, B, H, N, d,
                                           _stream_ptr(k.device))
    if st != _lib.FA_OK:
        raise FAError(st, "fa_bwd_preprocess")


def fa_bwd_dq(q, k, v, do, lse, workspace, dq, causal=False, scale=None, d_ready=False):
    """Phase 2 of fa_bwd: dQ (plus lse and D per query row in ``workspace``).
    ``d_ready``: the preprocess was given o_res (D is in the workspace)."""
    torch = _torch()
    B, H, N, d, ws = _bwd_common(k, [(q, "q"), (v, "v"), (do, "do"), (dq, "dq")], lse,
                                 workspace)
    with torch.cuda.device(k.device):
        st = _lib.load().fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                   lse.data_ptr(), workspace.data_ptr(), ws, dq.data_ptr(),
                                   B, H, N, d, int(bool(causal)), _scale(scale, d),
                                   int(bool(d_ready)), _stream_ptr(k.device))
    if st != _lib.FA_OK:
        raise FAError(st, "fa_bwd_dq")


def fa_bwd_dkdv(q, k, v, do, workspace, dk, dv, causal=False, scale=None):
    """Phase 3 of fa_bwd: dK and dV from q, k, v, dO and the workspace."""
    torch = _torch()
    B, H, N, d, ws = _bwd_common(k, [(q, "q"), (v, "v"), (do, "do"), (dk, "dk"), (dv, "dv")],
                                 None, workspace)
    with torch.cuda.device(k.device):
        st = _lib.load().fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                     workspace.data_ptr(), ws, dk.data_ptr(), dv.data_ptr(),
                                     B, H, N, d, int(bool(causal)), _scale(scale, d),
                                     _stream_ptr(k.device))
    if st != _lib.FA_OK:
        raise FAError(st, "fa_bwd_dkdv")


def fa_decode_workspace_size(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(_lib.load().fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d))


def fa_decode(q, k, v, causal: bool = False, scale: Optional[float] = None, out=None,
              lse=None, workspace=None):
    """bf16 decoding: q [B,H,Nq,d] (the last Nq positions), k and v [B,Hkv,Nk,d]
    (Hkv dividing H, (H // Hkv) * Nq <= 32). Returns (O [B,H,Nq,d], lse
    [B,H,Nq]). Calls fa_decode of libfa.so; ``workspace`` may be a uint8 device
    tensor of fa_decode_workspace_size(...) bytes."""
    torch = _torch()
    bf = torch.bfloat16
    _check(q, "q", bf)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(k, "k", bf, (B, Hkv, Nk, d), q.device)
    _check(v, "v", bf, (B, Hkv, Nk, d), q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check(out, "out", bf, q.shape, q.device)
    _check(lse, "lse", torch.float32, (B, H, Nq), q.device)
    if workspace is None:
        need = fa_decode_workspace_size(B, H, Hkv, Nq, Nk, d)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q.device)
    with torch.cuda.device(q.device):
        st = _lib.load().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), workspace.data_ptr(), ws_bytes, B, H, Hkv,
                                   Nq, Nk, d, int(bool(causal)), _scale(scale, d),
                                   _stream_ptr(q.device))
    if st != _lib.FA_OK:
        raise FAError(st, "fa_decode")
    return out, lse


def fa_decode_noalloc(q, k, v, causal: bool = False, scale: Optional[float] = None, out=None,
                      lse=None):
    """fa_decode with the library's fixed device buffer in place of a
    workspace (no device allocation inside the call; ``out`` and ``lse``
    are allocated here only when not given). Same results as fa_decode;
    problems whose partial results exceed the buffer raise FAError
    (FA_ERR_WORKSPACE). Calls that overlap on one GPU race. Calls
    fa_decode_noalloc of libfa.so."""
    torch = _torch()
    bf = torch.bfloat16
    _check(q, "q", bf)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(k, "k", bf, (B, Hkv, Nk, d), q.device)
    _check(v, "v", bf, (B, Hkv, Nk, d), q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check(out, "out", bf, q.shape, q.device)
    _check(lse, "lse", torch.float32, (B, H, Nq), q.device)
    with torch.cuda.device(q.device):
        st = _lib.load().fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           out.data_ptr(), lse.data_ptr(), B, H, Hkv, Nq, Nk, d,
                                           int(bool(causal)), _scale(scale, d),
                                           _stream_ptr(q.device))
    if st != _lib.FA_OK:
        raise FAError(st, "fa_decode_noalloc")
    return out, lse


def fa_fwd_rect(q, k, v, causal: bool = False, scale: Optional[float] = None, out=None,
                lse=None, o_res=None):
    """bf16 forward with Nq query rows against Nk keys: q [B,H,Nq,d], k and v
    [B,Hkv,Nk,d] (Hkv dividing H). Query row i sits at position Nk - Nq + i
    (bottom-right causal alignment). Returns (O [B,H,Nq,d], lse [B,H,Nq]).
    Calls fa_fwd_rect of libfa.so, or fa_fwd_train when ``o_res`` is given (as
    for fa_fwd)."""
    torch = _torch()
    bf = torch.bfloat16
    _check(q, "q", bf)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, Hkv, Nk, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(k, "k", bf, (B, Hkv, Nk, d), q.device)
    _check(v, "v", bf, (B, Hkv, Nk, d), q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check(out, "out", bf, q.shape, q.device)
    _check(lse, "lse", torch.float32, (B, H, Nq), q.device)
    entry = "fa_fwd_rect" if o_res is None else "fa_fwd_train"
    res = () if o_res is None else (_o_res_ptr(o_res, q),)
    with torch.cuda.device(q.device):
        st = getattr(_lib.load(), entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         out.data_ptr(), *res, lse.data_ptr(), B, H, Hkv, Nq,
                                         Nk, d, int(bool(causal)), _scale(scale, d),
                                         _stream_ptr(q.device))
    if st != _lib.FA_OK:
        raise FAError(st, entry)
    return out, lse


def fa_fwd_train(q, k, v, o_res, causal: bool = False, scale: Optional[float] = None,
                 out=None, lse=None):
    """Forward for training (fa_fwd_train of libfa.so): fa_fwd_rect that also
    stores O's rounding residual in ``o_res`` (bf16, q's shape). Returns
    (O, lse)."""
    if o_res is None:
        raise ValueError("fa_fwd_train needs o_res")
    return fa_fwd_rect(q, k, v, causal=causal, scale=scale, out=out, lse=lse, o_res=o_res)


def fa_bwd_train(q, k, v, o, o_res, do, lse, causal: bool = False,
                 scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None):
    """Backward for training (fa_bwd_train of libfa.so): the gradients of
    fa_fwd_train's output, with D formed from o and ``o_res``. Shapes as for
    fa_bwd_rect."""
    if o_res is None:
        raise ValueError("fa_bwd_train needs o_res")
    return fa_bwd_rect(q, k, v, o, do, lse, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv,
                       workspace=workspace, o_res=o_res)


def fa_fwd_fp8(q, k, v, descale_q: float = 1.0, descale_k: float = 1.0, descale_v: float = 1.0,
               causal: bool = False, scale: Optional[float] = None, out=None, lse=None):
    """Forward with e4m3 operands: q [B,H,Nq,d], k and v [B,Hkv,Nk,d] as
    torch.float8_e4m3fn (or their uint8 bytes), the real values being
    descale_x times the stored ones; d = 128. Rows aligned as in fa_fwd_rect.
    Returns (O [B,H,Nq,d] bf16, lse [B,H,Nq] fp32). Calls fa_fwd_fp8 of
    libfa.so."""
    torch = _torch()
    f8 = torch.float8_e4m3fn
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, Hkv, Nk, d]")
    dt = q.dtype if q.dtype in (f8, torch.uint8) else f8
    _check(q, "q", dt)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _check(k, "k", dt, (B, Hkv, Nk, d), q.device)
    _check(v, "v", dt, (B, Hkv, Nk, d), q.device)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check(out, "out", torch.bfloat16, (B, H, Nq, d), q.device)
    _check(lse, "lse", torch.float32, (B, H, Nq), q.device)
    with torch.cuda.device(q.device):
        st = _lib.load().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, Hkv, Nq, Nk, d, int(bool(causal)),
                                    _scale(scale, d), float(descale_q), float(descale_k),
                                    float(descale_v), _stream_ptr(q.device))
    if st != _lib.FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return out, lse


def fa_clock_probe(samples, sleep_units: int = 1, stream=None) -> None:
    """Measurement utility: enqueue on ``stream`` (a torch stream; default the
    current one) one wave that fills ``samples`` (an int64 device tensor
    [n, 2]) with (shader-clock counter, 100 MHz real-time counter) pairs,
    about sleep_units x 8128 shader clocks apart. Calls fa_clock_probe of
    libfa.so."""
    torch = _torch()
    if not isinstance(samples, torch.Tensor) or samples.dtype != torch.int64 or \
            samples.dim() != 2 or samples.shape[1] != 2 or not samples.is_contiguous():
        raise ValueError("samples must be a contiguous int64 tensor of shape [n, 2]")
    if samples.device.type != "cuda":
        raise ValueError("samples must be on a GPU")
    st = stream if stream is not None else torch.cuda.current_stream(samples.device)
    with torch.cuda.device(samples.device):
        rc = _lib.load().fa_clock_probe(samples.data_ptr(), samples.shape[0], int(sleep_units),
                                        st.cuda_stream)
    if rc != _lib.FA_OK:
        raise FAError(rc, "fa_clock_probe")


_AUTOGRAD_FN = None


def _autograd_fn():
    """torch.autograd.Function over fa_fwd_train / fa_bwd_train (built once)."""
    global _AUTOGRAD_FN
    if _AUTOGRAD_FN is None:
        torch = _torch()

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, causal, scale):
                o_res = torch.empty_like(q)
                o, lse = fa_fwd_rect(q, k, v, causal=causal, scale=scale, o_res=o_res)
                ctx.save_for_backward(q, k, v, o, o_res, lse)
                ctx.causal, ctx.scale = causal, scale
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, o_res, lse = ctx.saved_tensors
                dq, dk, dv = fa_bwd_rect(q, k, v, o, do.contiguous(), lse, causal=ctx.causal,
                                         scale=ctx.scale, o_res=o_res)
                return dq, dk, dv, None, None

        _AUTOGRAD_FN = _Attention
    return _AUTOGRAD_FN


def fa_attention(q, k, v, causal: bool = False, scale: Optional[float] = None):
    """Attention with autograd: O = softmax(scale Q K^T) V for bf16 q [B,H,Nq,d]
    and k, v [B,Hkv,Nk,d] on a GPU (Hkv dividing H; query row i at position
    Nk - Nq + i, bottom-right causal). The forward is fa_fwd_train (fa_fwd_rect
    keeping O's rounding residual); the gradient of a loss with respect to q,
    k and v is fa_bwd_train, fed the saved O, its residual and the logsumexp.
    Both run in libfa.so."""
    return _autograd_fn().apply(q, k, v, bool(causal), _scale(scale, q.shape[-1]))
