"""GPTQ per-layer quantization solver for AMD MI355X (gfx950).

Python face of libgptq_mi355x.so.  The functions below mirror the C ABI of
``include/gptq.h`` one to one (same names without the ``gptq_`` prefix) and
only marshal torch tensors (device memory) and the current HIP stream into
the library; ``quantize`` chains the four calls for one layer.

Import is cheap: the shared library is loaded on first use, and a missing
library raises instead of falling back to anything else.
"""
from __future__ import annotations

import contextlib
import ctypes

from . import _lib
from ._lib import (  # noqa: F401
    BF16, F16, F32, Config, GPTQError, InvalidArgument, NonFinite, NotPositiveDefinite,
    Unsupported, WorkspaceError, make_config, load, version, status_string,
)

__all__ = ["hessian_accumulate", "hessian_accumulate_timed", "hessian_accumulate_noalloc", "prepare_hinv", "quantize_layer", "prepare_hinv_factored", "quantize_layer_factored", "factored_supported", "pack", "quantize",
           "pack_permuted", "dequant_matmul", "dequant_max_groups", "gather_columns", "packed_words_per_row", "make_config",
           "Config", "load"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _alloc_on(stream):
    """Allocations made inside belong to ``stream`` (the caching allocator
    then never hands their memory to other work before the stream's queued
    kernels are done with it); torch's current stream when None."""
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _workspace(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def hessian_accumulate(H, X, stream=None):
    """H (d_in x d_in float64, upper triangle) += 2 X^T X; X is tokens x d_in."""
    lib = load()
    torch = _torch()
    _require_cuda(H, X)
    if H.dtype != torch.float64 or not H.is_contiguous():
        raise TypeError("H must be a contiguous float64 tensor")
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    n_tok, d_in = X.shape
    if H.shape != (d_in, d_in):
        raise ValueError("H must be d_in x d_in")
    nws = lib.gptq_hessian_workspace(n_tok, d_in)
    with _alloc_on(stream):
        ws = _workspace(nws, H.device)
    st = lib.gptq_hessian_accumulate(_ptr(H), _ptr(X), _dtype_code(X), n_tok, d_in, X.stride(0),
                                     _ptr(ws), nws, _stream(stream))
    _lib.check(st, "gptq_hessian_accumulate")
    return H


def hessian_accumulate_timed(H, X, stream=None):
    """hessian_accumulate with HIP events around each Hessian product launch
    (synchronous); returns (mean launch ms, number of launches)."""
    lib = load()
    torch = _torch()
    _require_cuda(H, X)
    if H.dtype != torch.float64 or not H.is_contiguous():
        raise TypeError("H must be a contiguous float64 tensor")
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    n_tok, d_in = X.shape
    if H.shape != (d_in, d_in):
        raise ValueError("H must be d_in x d_in")
    nws = lib.gptq_hessian_workspace(n_tok, d_in)
    with _alloc_on(stream):
        ws = _workspace(nws, H.device)
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    st = lib.gptq_hessian_accumulate_timed(_ptr(H), _ptr(X), _dtype_code(X), n_tok, d_in, X.stride(0),
                                           _ptr(ws), nws, _stream(stream), ctypes.byref(ms), ctypes.byref(n))
    _lib.check(st, "gptq_hessian_accumulate_timed")
    return ms.value, n.value


def hessian_accumulate_noalloc(H, X, stream=None):
    """hessian_accumulate through the allocation-free entry point: no
    workspace (the library's fixed per-GPU scratch array instead)."""
    lib = load()
    torch = _torch()
    _require_cuda(H, X)
    if H.dtype != torch.float64 or not H.is_contiguous():
        raise TypeError("H must be a contiguous float64 tensor")
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    n_tok, d_in = X.shape
    if H.shape != (d_in, d_in):
        raise ValueError("H must be d_in x d_in")
    st = lib.gptq_hessian_accumulate_noalloc(_ptr(H), _ptr(X), _dtype_code(X), n_tok, d_in, X.stride(0),
                                             _stream(stream))
    _lib.check(st, "gptq_hessian_accumulate_noalloc")
    return H


def _prepare(name, H, cfg, perm, workspace, stream):
    lib = load()
    torch = _torch()
    _require_cuda(H)
    if H.dtype != torch.float64 or not H.is_contiguous() or H.dim() != 2 or H.shape[0] != H.shape[1]:
        raise TypeError("H must be a square contiguous float64 tensor")
    d = H.shape[0]
    nws = getattr(lib, name + "_workspace")(d)
    with _alloc_on(stream):
        if perm is None:
            perm = torch.empty(d, dtype=torch.int32, device=H.device)
        ws = workspace if workspace is not None else _workspace(nws, H.device)
    st = getattr(lib, name)(_ptr(H), d, ctypes.byref(cfg), _ptr(perm), _ptr(ws),
                            ws.numel() if ws is not None else 0, _stream(stream))
    _lib.check(st, name)
    return perm


def prepare_hinv(H, cfg: Config, perm=None, workspace=None, stream=None):
    """In place H -> U (upper Cholesky factor of the damped, permuted inverse); returns perm."""
    return _prepare("gptq_prepare_hinv", H, cfg, perm, workspace, stream)


def prepare_hinv_factored(H, cfg: Config, perm=None, workspace=None, stream=None):
    """In place H -> F, the factored form read by quantize_layer_factored (d_in a multiple of 128); returns perm."""
    return _prepare("gptq_prepare_hinv_factored", H, cfg, perm, workspace, stream)


def n_groups(d_in: int, group_size: int) -> int:
    return -(-d_in // group_size) if group_size > 0 else 1


def quantize_layer(W, U, perm, cfg: Config, want_w_hat=True, want_row_loss=True, workspace=None,
                   out=None, stream=None):
    """Column sweep; returns dict(codes, scales, zeros, g_idx[, w_hat][, row_loss]) in original order."""
    return _quantize("gptq_quantize_layer", W, U, perm, cfg, want_w_hat, want_row_loss, workspace, out, stream)


def quantize_layer_factored(W, F, perm, cfg: Config, want_w_hat=True, want_row_loss=True, workspace=None,
                            out=None, stream=None):
    """The column sweep given F from prepare_hinv_factored; the same outputs as quantize_layer."""
    return _quantize("gptq_quantize_layer_factored", W, F, perm, cfg, want_w_hat, want_row_loss, workspace, out,
                     stream)


def _quantize(name, W, U, perm, cfg, want_w_hat, want_row_loss, workspace, out, stream):
    lib = load()
    torch = _torch()
    _require_cuda(W, U, perm)
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be 2-D with unit column stride")
    d_out, d_in = W.shape
    if U.dtype != torch.float64 or U.shape != (d_in, d_in) or not U.is_contiguous():
        raise TypeError("U must be a contiguous d_in x d_in float64 tensor")
    if perm.dtype != torch.int32 or perm.numel() != d_in:
        raise TypeError("perm must be int32 of length d_in")
    dev = W.device
    ng = n_groups(d_in, cfg.group_size)
    nws = getattr(lib, name + "_workspace")(d_out, d_in, ctypes.byref(cfg))
    if nws == 0:
        raise InvalidArgument(_lib.ERR_INVALID_ARG, name + "_workspace", "invalid or unsupported shape or config")
    with _alloc_on(stream):
        if out is None:
            out = dict(codes=torch.empty((d_out, d_in), dtype=torch.uint8, device=dev),
                       scales=torch.empty((ng, d_out), dtype=torch.float32, device=dev),
                       zeros=torch.empty((ng, d_out), dtype=torch.float32, device=dev),
                       g_idx=torch.empty(d_in, dtype=torch.int32, device=dev))
            if want_w_hat:
                out["w_hat"] = torch.empty((d_out, d_in), dtype=torch.float32, device=dev)
            if want_row_loss:
                out["row_loss"] = torch.empty(d_out, dtype=torch.float64, device=dev)
        ws = workspace if workspace is not None else _workspace(nws, dev)
    st = getattr(lib, name)(_ptr(W), _dtype_code(W), d_out, d_in, W.stride(0), _ptr(U), _ptr(perm),
                            ctypes.byref(cfg), _ptr(out["codes"]), _ptr(out["scales"]), _ptr(out["zeros"]),
                            _ptr(out["g_idx"]), _ptr(out.get("w_hat")), _ptr(out.get("row_loss")),
                            _ptr(ws), ws.numel(), _stream(stream))
    _lib.check(st, name)
    return out


def packed_words_per_row(d_in: int, bits: int) -> int:
    return int(load().gptq_packed_words_per_row(d_in, bits))


def pack(codes, bits: int, out=None, stream=None):
    """codes (d_out x d_in uint8) -> packed uint32 words, per-row little-endian bit stream."""
    lib = load()
    torch = _torch()
    _require_cuda(codes)
    if codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise TypeError("codes must be contiguous uint8")
    d_out, d_in = codes.shape
    wpr = packed_words_per_row(d_in, bits)
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((d_out, wpr), dtype=torch.int32, device=codes.device)
    st = lib.gptq_pack(_ptr(codes), d_out, d_in, bits, _ptr(out), _stream(stream))
    _lib.check(st, "gptq_pack")
    return out


def pack_permuted(codes, bits: int, perm, out=None, stream=None):
    """Pack with stream position k of every row holding column perm[k]."""
    lib = load()
    torch = _torch()
    _require_cuda(codes, perm)
    if codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise TypeError("codes must be contiguous uint8")
    d_out, d_in = codes.shape
    if perm.dtype != torch.int32 or perm.numel() != d_in or not perm.is_contiguous():
        raise TypeError("perm must be contiguous int32 of length d_in")
    wpr = packed_words_per_row(d_in, bits)
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((d_out, wpr), dtype=torch.int32, device=codes.device)
    st = lib.gptq_pack_permuted(_ptr(codes), d_out, d_in, bits, _ptr(perm), _ptr(out), _stream(stream))
    _lib.check(st, "gptq_pack_permuted")
    return out


def dequant_max_groups() -> int:
    return int(load().gptq_dequant_max_groups())


def dequant_matmul(X, packed, bits: int, scales, zeros, *, g_idx=None, perm=None, group_size: int = -1,
                   out=None, stream=None):
    """Y = X W_hat^T (float32, tokens x d_out) straight from packed words.

    X: tokens x d_in (bf16 / f16 / f32, unit column stride); packed: d_out x
    words-per-row int32/uint32 words; scales, zeros: [n_groups][d_out] float32.
    g_idx (original order) or perm (words from pack_permuted) select the
    column order, as in gptq_dequant_matmul.  With perm and two or more
    tokens, dequant_matmul(gather_columns(X, perm), packed, ...) without perm
    is the faster form (the matrix-core routes read activations in order).
    """
    lib = load()
    torch = _torch()
    _require_cuda(X, packed, scales, zeros, g_idx, perm)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    n_tok, d_in = X.shape
    if packed.dim() != 2 or not packed.is_contiguous() or packed.element_size() != 4:
        raise TypeError("packed must be a contiguous 2-D tensor of 32-bit words")
    d_out = packed.shape[0]
    if packed.shape[1] != packed_words_per_row(d_in, bits):
        raise ValueError("packed has the wrong number of words per row")
    for name, t in (("scales", scales), ("zeros", zeros)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 2 or t.shape[1] != d_out:
            raise TypeError(f"{name} must be contiguous float32 [n_groups][d_out]")
    for name, t in (("g_idx", g_idx), ("perm", perm)):
        if t is not None and (t.dtype != torch.int32 or t.numel() != d_in or not t.is_contiguous()):
            raise TypeError(f"{name} must be contiguous int32 of length d_in")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((n_tok, d_out), dtype=torch.float32, device=X.device)
    if out.dtype != torch.float32 or out.dim() != 2 or out.stride(1) != 1 or out.shape != (n_tok, d_out):
        raise TypeError("out must be float32 tokens x d_out with unit column stride")
    st = lib.gptq_dequant_matmul(_ptr(X), _dtype_code(X), n_tok, d_in, X.stride(0), _ptr(packed), bits,
                                 _ptr(scales), _ptr(zeros), scales.shape[0], _ptr(g_idx), _ptr(perm),
                                 int(group_size), d_out, _ptr(out), out.stride(0), _stream(stream))
    _lib.check(st, "gptq_dequant_matmul")
    return out


def gather_columns(X, perm, out=None, stream=None):
    """Xg[t][k] = X[t][perm[k]] (the activations in quantization order)."""
    lib = load()
    torch = _torch()
    _require_cuda(X, perm)
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    n_tok, d_in = X.shape
    if perm.dtype != torch.int32 or perm.numel() != d_in or not perm.is_contiguous():
        raise TypeError("perm must be contiguous int32 of length d_in")
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((n_tok, d_in), dtype=X.dtype, device=X.device)
    if out.dtype != X.dtype or out.shape != X.shape or out.stride(1) != 1:
        raise TypeError("out must match X in dtype and shape, with unit column stride")
    st = lib.gptq_gather_columns(_ptr(X), _dtype_code(X), n_tok, d_in, X.stride(0), _ptr(perm), _ptr(out),
                                 out.stride(0), _stream(stream))
    _lib.check(st, "gptq_gather_columns")
    return out


def factored_supported(d_out: int, d_in: int, cfg: Config) -> bool:
    """Whether prepare_hinv_factored / quantize_layer_factored take this shape and config."""
    lib = load()
    return (lib.gptq_prepare_hinv_factored_workspace(d_in) != 0 and
            lib.gptq_quantize_layer_factored_workspace(d_out, d_in, ctypes.byref(cfg)) != 0)


def quantize(W, *, X=None, H=None, cfg: Config | None = None, packed=True, factored=None, stream=None):
    """One layer end to end: Hessian (from X unless H is given), prepare, sweep, pack.

    factored: None takes the factored form (prepare_hinv_factored,
    quantize_layer_factored) where it is supported, else U; True or False
    forces one of them.  Returns the dict of quantize_layer plus ``perm``
    and (if packed) ``packed``.  H, when given, is consumed (overwritten).
    """
    torch = _torch()
    cfg = cfg or make_config()
    d_out, d_in = W.shape
    if factored is None:
        factored = factored_supported(d_out, d_in, cfg)
    if H is None:
        if X is None:
            raise ValueError("give X or H")
        with _alloc_on(stream):
            H = torch.zeros((d_in, d_in), dtype=torch.float64, device=W.device)
        hessian_accumulate(H, X, stream=stream)
    if factored:
        perm = prepare_hinv_factored(H, cfg, stream=stream)
        out = quantize_layer_factored(W, H, perm, cfg, stream=stream)
    else:
        perm = prepare_hinv(H, cfg, stream=stream)
        out = quantize_layer(W, H, perm, cfg, stream=stream)
    out["perm"] = perm
    if packed:
        out["packed"] = pack(out["codes"], cfg.bits, stream=stream)
    return out
