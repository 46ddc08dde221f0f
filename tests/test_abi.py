"""The C-ABI boundary without a GPU: header, exported symbols, argument checks.

Only calls that the library rejects during validation (before any HIP call)
or that are empty no-ops are made here; nothing is launched.
"""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from exact_attention_41_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from exact_attention_41_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    """Every function that a header under include/ declares."""
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_compiles_as_c_and_cpp(tmp_path):
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++11")):
        src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
        src.write_text('#include "fa.h"\n#include "fa_measure.h"\n'
                       'int main(void){ return (int)FA_OK; }\n')
        cc = "gcc" if lang == "c" else "g++"
        res = subprocess.run([cc, std, "-Wall", "-Werror", "-fsyntax-only", "-I",
                              os.path.join(ROOT, "include"), str(src)],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(fa_[a-z0-9_]+)\b", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.fa_status_str(code).decode() == name
    assert lib.fa_status_str(99).decode() == "FA_ERR_UNKNOWN"


def test_workspace_size(lib):
    rows = 4 * 16 * 4096
    assert lib.fa_bwd_workspace_size(4, 16, 4096, 128) >= rows * (4 + 2 * 2 * 128)
    assert lib.fa_bwd_workspace_size(4, 16, 4096, 128) % 256 == 0
    assert lib.fa_bwd_workspace_size(4, 16, 4096, 64) < lib.fa_bwd_workspace_size(4, 16, 4096, 128)
    assert lib.fa_bwd_workspace_size(4, 16, 4096, 96) == 0
    assert lib.fa_bwd_workspace_size(0, 16, 4096, 128) == 0
    assert lib.fa_bwd_workspace_size(-1, 16, 4096, 128) == 0


# Fake, never-dereferenced "device" addresses for validation-only calls.
A = 0x100000          # 16-byte aligned
MIS = 0x100008        # 8-byte aligned only


def fwd(lib, entry, q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=64, d=64, causal=0, scale=0.125):
    return getattr(lib, entry)(q, k, v, o, lse, B, H, N, d, causal, scale, None)


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f32"])
def test_forward_rejects_bad_arguments(lib, entry):
    assert fwd(lib, entry, q=None) == INVALID
    assert fwd(lib, entry, lse=None) == INVALID
    assert fwd(lib, entry, B=-1) == INVALID
    assert fwd(lib, entry, N=-5) == INVALID
    assert fwd(lib, entry, scale=float("nan")) == INVALID
    assert fwd(lib, entry, scale=float("inf")) == INVALID
    assert fwd(lib, entry, scale=-0.5) == INVALID
    # 0 too: a masked score is -inf before scaling, and -inf * 0 is NaN
    assert fwd(lib, entry, scale=0.0) == INVALID
    assert fwd(lib, entry, scale=-0.0) == INVALID
    assert fwd(lib, entry, d=96) == UNSUPPORTED
    assert fwd(lib, entry, d=512) == UNSUPPORTED
    if entry == "fa_fwd_f32":
        assert fwd(lib, entry, d=256) == UNSUPPORTED     # d = 256: bf16 forward only
    assert fwd(lib, entry, q=MIS) == UNSUPPORTED
    assert fwd(lib, entry, o=MIS) == UNSUPPORTED
    assert fwd(lib, entry, lse=A + 2) == UNSUPPORTED
    assert fwd(lib, entry, N=(1 << 26) + 1) == UNSUPPORTED
    assert fwd(lib, entry, B=1 << 16, H=1 << 16, N=64) == UNSUPPORTED


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f32"])
def test_forward_empty_problem_is_a_no_op(lib, entry):
    # Empty sizes return before any pointer is looked at.
    assert fwd(lib, entry, q=None, k=None, v=None, o=None, lse=None, B=0) == OK
    assert fwd(lib, entry, q=None, k=None, v=None, o=None, lse=None, H=0) == OK
    assert fwd(lib, entry, q=None, k=None, v=None, o=None, lse=None, N=0) == OK


def bwd(lib, ws=0x200000, ws_bytes=None, B=1, H=2, N=100, d=128, **ptrs):
    p = dict(q=A, k=A, v=A, o=A, do=A, lse=A, dq=A, dk=A, dv=A)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d)
    return lib.fa_bwd(p["q"], p["k"], p["v"], p["o"], p["do"], p["lse"], p["dq"], p["dk"],
                      p["dv"], ws, ws_bytes, B, H, N, d, 1, 0.088, None)


def test_backward_rejects_bad_arguments(lib):
    assert bwd(lib, do=None) == INVALID
    assert bwd(lib, dv=None) == INVALID
    assert bwd(lib, H=-2) == INVALID
    assert bwd(lib, d=32) == UNSUPPORTED
    assert bwd(lib, dk=MIS) == UNSUPPORTED
    assert bwd(lib, ws=None) == WORKSPACE
    assert bwd(lib, ws=MIS) == WORKSPACE
    assert bwd(lib, ws=0x200000 + 128) == WORKSPACE
    assert bwd(lib, ws_bytes=lib.fa_bwd_workspace_size(1, 2, 100, 128) - 1) == WORKSPACE
    assert bwd(lib, B=0, ws=None, ws_bytes=0) == OK


def test_grouped_heads_arguments(lib):
    """fa_fwd_gqa / fa_bwd_gqa: Hkv must be >= 1 and divide H."""
    def f(Hkv, H=4, **kw):
        return lib.fa_fwd_gqa(A, A, A, A, A, 1, H, Hkv, 64, 64, 0, 0.125, None)
    assert f(0) == INVALID
    assert f(-1) == INVALID
    assert f(3) == INVALID
    assert f(8) == INVALID
    assert lib.fa_fwd_gqa(None, A, A, A, A, 1, 4, 2, 64, 64, 0, 0.125, None) == INVALID
    assert lib.fa_fwd_gqa(A, A, A, A, A, 1, 4, 2, 64, 96, 0, 0.125, None) == UNSUPPORTED
    assert lib.fa_fwd_gqa(A, A, A, A, A, 0, 4, 2, 64, 64, 0, 0.125, None) == OK
    assert lib.fa_bwd_gqa_workspace_size(2, 32, 8, 4096, 128) > 0
    # d = 256: twice the images of d = 128 (one per 128-column part)
    assert lib.fa_bwd_gqa_workspace_size(2, 32, 8, 4096, 256) > \
        lib.fa_bwd_gqa_workspace_size(2, 32, 8, 4096, 128)
    assert lib.fa_bwd_gqa_workspace_size(2, 32, 5, 4096, 128) == 0
    assert lib.fa_bwd_gqa_workspace_size(2, 32, 0, 4096, 128) == 0
    assert lib.fa_bwd_gqa_workspace_size(4, 16, 16, 4096, 128) == \
        lib.fa_bwd_workspace_size(4, 16, 4096, 128)
    # fewer K/V heads: smaller workspace (one K image per K/V head)
    assert lib.fa_bwd_gqa_workspace_size(4, 16, 4, 4096, 128) < \
        lib.fa_bwd_workspace_size(4, 16, 4096, 128)
    ws = lib.fa_bwd_gqa_workspace_size(1, 4, 2, 100, 128)

    def b(Hkv=2, ws_bytes=ws, **kw):
        return lib.fa_bwd_gqa(A, A, A, A, A, A, A, A, A, 0x200000, ws_bytes, 1, 4, Hkv, 100, 128,
                              1, 0.088, None)
    assert b(Hkv=3) == INVALID
    assert b(Hkv=0) == INVALID
    assert b(ws_bytes=ws - 1) == WORKSPACE


def test_decode_arguments(lib):
    ws = lib.fa_decode_workspace_size(2, 8, 2, 4, 1000, 128)
    assert ws > 0 and ws % 256 == 0
    assert lib.fa_decode_workspace_size(2, 8, 2, 5, 4, 128) == 0      # Nq > Nk
    assert lib.fa_decode_workspace_size(2, 8, 3, 1, 100, 128) == 0     # Hkv does not divide H
    assert lib.fa_decode_workspace_size(1, 64, 1, 1, 100, 128) == 0    # 64 rows per K/V head
    assert lib.fa_decode_workspace_size(2, 8, 2, 4, 1000, 256) > ws      # d = 256 is supported
    assert lib.fa_decode_workspace_size(2, 8, 2, 4, 1000, 512) == 0

    def dec(B=2, H=8, Hkv=2, Nq=4, Nk=1000, d=128, ws_bytes=ws, o=A, wsp=0x200000, scale=0.1):
        return lib.fa_decode(A, A, A, o, A, wsp, ws_bytes, B, H, Hkv, Nq, Nk, d, 1, scale, None)
    assert dec(Hkv=3) == INVALID
    assert dec(Nq=1001) == INVALID
    assert dec(scale=float("nan")) == INVALID
    assert dec(scale=0.0) == INVALID
    assert dec(o=None) == INVALID
    assert dec(d=96) == UNSUPPORTED
    assert dec(H=64, Hkv=1, Nq=1) == UNSUPPORTED
    assert dec(o=MIS) == UNSUPPORTED
    assert dec(wsp=None) == WORKSPACE
    assert dec(ws_bytes=ws - 1) == WORKSPACE
    assert dec(B=0, wsp=None, ws_bytes=0) == OK
    assert dec(Nq=0, wsp=None, ws_bytes=0) == OK


def test_decode_noalloc_arguments(lib):
    """fa_decode_noalloc validates like fa_decode (no workspace argument) and
    refuses problems whose partial results exceed its fixed 40 MiB buffer,
    all before any HIP call."""
    def dec(B=2, H=8, Hkv=2, Nq=4, Nk=1000, d=128, o=A, scale=0.1):
        return lib.fa_decode_noalloc(A, A, A, o, A, B, H, Hkv, Nq, Nk, d, 1, scale, None)
    assert dec(Hkv=3) == INVALID
    assert dec(Nq=1001) == INVALID
    assert dec(scale=0.0) == INVALID
    assert dec(o=None) == INVALID
    assert dec(d=96) == UNSUPPORTED
    assert dec(o=MIS) == UNSUPPORTED
    assert dec(B=0) == OK
    assert dec(Nq=0) == OK
    # 2047 K/V heads at d = 128: about 65 MiB of partial results
    assert lib.fa_decode_workspace_size(2047, 1, 1, 1, 64, 128) > 40 << 20
    assert dec(B=2047, H=1, Hkv=1, Nq=1, Nk=64) == WORKSPACE


def test_rect_forward_arguments(lib):
    def f(B=1, H=2, Hkv=1, Nq=100, Nk=300, d=128, q=A, scale=0.1):
        return lib.fa_fwd_rect(q, A, A, A, A, B, H, Hkv, Nq, Nk, d, 1, scale, None)
    assert f(Nk=-1) == INVALID
    assert f(Nk=0) == INVALID
    assert f(Hkv=3) == INVALID
    assert f(q=None) == INVALID
    assert f(scale=0.0) == INVALID
    assert f(d=256 + 32) == UNSUPPORTED
    assert f(Nk=(1 << 26) + 1) == UNSUPPORTED
    assert f(Nq=0, Nk=0, q=None) == OK          # nothing to compute
    assert f(B=0) == OK


def test_rect_backward_arguments(lib):
    """fa_bwd_rect: sizes of the rectangular backward and its argument errors."""
    ws = lib.fa_bwd_rect_workspace_size(1, 4, 2, 100, 300, 128)
    assert ws > 0 and ws % 256 == 0
    assert lib.fa_bwd_rect_workspace_size(2, 32, 8, 4096, 4096, 128) == \
        lib.fa_bwd_gqa_workspace_size(2, 32, 8, 4096, 128)
    # more keys: more K images; more query rows: more Q/dO images and statistics
    assert lib.fa_bwd_rect_workspace_size(1, 4, 2, 100, 3000, 128) > ws
    assert lib.fa_bwd_rect_workspace_size(1, 4, 2, 1000, 300, 128) > ws
    assert lib.fa_bwd_rect_workspace_size(1, 4, 2, 0, 300, 128) == 0
    assert lib.fa_bwd_rect_workspace_size(1, 4, 2, 100, 0, 128) == 0
    assert lib.fa_bwd_rect_workspace_size(1, 4, 3, 100, 300, 128) == 0
    assert lib.fa_bwd_rect_workspace_size(1, 4, 2, 100, 300, 256) > ws
    assert lib.fa_bwd_rect_workspace_size(1, 4, 2, 100, 300, 512) == 0

    def b(B=1, H=4, Hkv=2, Nq=100, Nk=300, d=128, ws_bytes=ws, wsp=0x200000, dk=A):
        return lib.fa_bwd_rect(A, A, A, A, A, A, A, dk, A, wsp, ws_bytes, B, H, Hkv, Nq, Nk, d,
                               1, 0.088, None)
    assert b(Nk=-1) == INVALID
    assert b(Nk=0) == INVALID                   # query rows but no keys
    assert b(Nq=0) == INVALID                   # keys whose gradients would be left unwritten
    assert b(Hkv=3) == INVALID
    assert b(dk=None) == INVALID
    assert b(d=512) == UNSUPPORTED
    assert b(d=96) == UNSUPPORTED
    assert b(Nk=(1 << 26) + 1) == UNSUPPORTED
    assert b(dk=MIS) == UNSUPPORTED
    assert b(ws_bytes=ws - 1) == WORKSPACE
    assert b(wsp=None) == WORKSPACE
    assert b(Nq=0, Nk=0, wsp=None, ws_bytes=0) == OK
    assert b(B=0, wsp=None, ws_bytes=0) == OK


def test_training_entry_points_arguments(lib):
    """fa_fwd_train / fa_bwd_train: fa_fwd_rect / fa_bwd_rect plus the
    rounding residual of O, which they need (NULL is an argument error)."""
    def f(o_res=A, q=A, B=1, H=2, Hkv=1, Nq=100, Nk=300, d=128):
        return lib.fa_fwd_train(q, A, A, A, o_res, A, B, H, Hkv, Nq, Nk, d, 1, 0.1, None)
    assert f(o_res=None) == INVALID
    assert f(q=None) == INVALID
    assert f(o_res=MIS) == UNSUPPORTED
    assert f(Hkv=3) == INVALID
    assert f(d=96) == UNSUPPORTED
    assert f(o_res=None, B=0) == OK                 # nothing to compute
    ws = lib.fa_bwd_rect_workspace_size(1, 2, 1, 100, 300, 128)

    def b(o_res=A, ws_bytes=ws, wsp=0x200000, B=1, Nq=100, Nk=300, dk=A):
        return lib.fa_bwd_train(A, A, A, A, o_res, A, A, A, dk, A, wsp, ws_bytes, B, 2, 1, Nq,
                                Nk, 128, 1, 0.088, None)
    assert b(o_res=None) == INVALID
    assert b(o_res=MIS) == UNSUPPORTED
    assert b(dk=None) == INVALID
    assert b(ws_bytes=ws - 1) == WORKSPACE
    assert b(Nq=0) == INVALID
    assert b(o_res=None, B=0, wsp=None, ws_bytes=0) == OK


def test_python_binding_refuses_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    import exact_attention_41_amd as fa
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(x, x, x)
    with pytest.raises(TypeError):
        fa.fa_fwd(x.float(), x.float(), x.float())


def test_binding_checks_caller_workspaces():
    """A caller's workspace must be a contiguous tensor on the inputs' device:
    its byte count is what the library is told it may write."""
    torch = pytest.importorskip("torch")
    import exact_attention_41_amd as fa
    cpu = torch.device("cpu")
    ws = torch.zeros(64, dtype=torch.uint8)
    assert fa._check_workspace(ws, cpu) == 64
    assert fa._check_workspace(torch.zeros(8, dtype=torch.float32), cpu) == 32
    with pytest.raises(ValueError):
        fa._check_workspace(ws[::2], cpu)                    # not contiguous
    with pytest.raises(ValueError):
        fa._check_workspace(ws, torch.device("cuda", 0))     # another device
    with pytest.raises(TypeError):
        fa._check_workspace(bytearray(64), cpu)


def test_backward_phases_reject_bad_arguments(lib):
    ws = lib.fa_bwd_workspace_size(1, 2, 100, 128)
    W = 0x200000     # 256-byte aligned fake workspace
    assert lib.fa_bwd_preprocess(None, A, A, A, None, A, W, ws, 1, 2, 100, 128, None) == INVALID
    assert lib.fa_bwd_preprocess(A, A, A, None, None, A, W, ws, 1, 2, 100, 128, None) == INVALID
    assert lib.fa_bwd_preprocess(A, A, A, A, None, A, W, ws - 4, 1, 2, 100, 128, None) == WORKSPACE
    assert lib.fa_bwd_preprocess(A, A, A, A, None, A, W + 16, ws, 1, 2, 100, 128, None) == WORKSPACE
    assert lib.fa_bwd_preprocess(A, MIS, A, A, None, A, W, ws, 1, 2, 100, 128, None) == UNSUPPORTED
    assert lib.fa_bwd_preprocess(A, A, A, MIS, None, A, W, ws, 1, 2, 100, 128, None) == UNSUPPORTED
    assert lib.fa_bwd_preprocess(A, A, A, A, MIS, A, W, ws, 1, 2, 100, 128, None) == UNSUPPORTED
    assert lib.fa_bwd_dq(A, A, A, A, None, W, ws, A, 1, 2, 100, 128, 1, 0.1, 0, None) == INVALID
    assert lib.fa_bwd_dq(A, A, A, A, A, W, ws, MIS, 1, 2, 100, 128, 1, 0.1, 0, None) == UNSUPPORTED
    assert lib.fa_bwd_dq(A, A, A, A, A, W, ws, A, 1, 2, 100, 96, 1, 0.1, 0, None) == UNSUPPORTED
    assert lib.fa_bwd_dq(A, A, A, A, A, W, ws, A, 0, 2, 100, 128, 1, 0.1, 0, None) == OK
    assert lib.fa_bwd_dkdv(A, A, A, A, W, ws, A, None, 1, 2, 100, 128, 1, 0.1, None) == INVALID
    assert lib.fa_bwd_dkdv(A, A, None, A, W, ws, A, A, 1, 2, 100, 128, 1, 0.1, None) == INVALID
    assert lib.fa_bwd_dkdv(A, A, A, A, None, ws, A, A, 1, 2, 100, 128, 1, 0.1, None) == WORKSPACE
    assert lib.fa_bwd_dkdv(A, A, A, A, W, ws, A, A, 1, 2, 100, 128, 1, -1.0, None) == INVALID
    assert lib.fa_bwd_dq(A, A, A, A, A, W, ws, A, 1, 2, 100, 128, 1, 0.0, 0, None) == INVALID


def test_fp8_forward_arguments(lib):
    def f(B=1, H=2, Hkv=1, Nq=100, Nk=300, d=128, q=A, scale=0.1, dq=0.01, dk=0.01, dv=0.01):
        return lib.fa_fwd_fp8(q, A, A, A, A, B, H, Hkv, Nq, Nk, d, 1, scale, dq, dk, dv, None)
    assert f(dq=0.0) == INVALID
    assert f(dk=-1.0) == INVALID
    assert f(dv=float("inf")) == INVALID
    assert f(dq=float("nan")) == INVALID
    assert f(Nk=-1) == INVALID
    assert f(Nk=0) == INVALID
    assert f(Hkv=3) == INVALID
    assert f(q=None) == INVALID
    assert f(d=64) == UNSUPPORTED
    assert f(d=256) == UNSUPPORTED
    assert f(q=MIS) == UNSUPPORTED
    assert f(B=0) == OK


def test_clock_probe_arguments(lib):
    """fa_clock_probe validates before launching (n = 0 launches nothing)."""
    import ctypes
    f = lib.fa_clock_probe
    assert f(None, 0, 1, None) == OK
    assert f(A, -1, 1, None) == INVALID
    assert f(A, 4, -1, None) == INVALID
    assert f(None, 4, 1, None) == INVALID
    assert f(A + 8, 4, 1, None) == UNSUPPORTED
    assert f(A, (1 << 20) + 1, 1, None) == UNSUPPORTED
    assert f(A, 4, 1025, None) == UNSUPPORTED
    assert isinstance(ctypes.c_int(f(A, 0, 0, None)).value, int)
