"""Python binding of libtsa, the MI355X tile-sparse attention library.

Thin ctypes marshalling over the C ABI declared in include/tsa.h: every
function takes torch tensors that live on the GPU, passes their device
pointers and the current HIP stream to the library, and raises TsaError on a
non-zero status.  Names are those of the C entry points without the `tsa_`
prefix.  There is no CPU fallback: if libtsa.so is missing the first call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtsa.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP = range(5)
DTYPE_F32, DTYPE_BF16 = 0, 1
OP_ATTENTION_FWD, OP_MASK_COMPACT, OP_PREDICT_MASK, OP_ATTENTION_BWD = 0, 1, 2, 3


class TsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"tsa status {status}: {detail}")
        self.status = status
        self.detail = detail


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d", ctypes.c_int32), ("M", ctypes.c_int32), ("N", ctypes.c_int32),
                ("dtype", ctypes.c_int)]


class MaskgenParams(ctypes.Structure):
    _fields_ = [("state0", ctypes.c_uint64), ("thr_near", ctypes.c_uint32),
                ("thr_far", ctypes.c_uint32), ("frame_tokens", ctypes.c_int32),
                ("frame_radius", ctypes.c_int32), ("force_diag", ctypes.c_int32)]


class StructuredParams(ctypes.Structure):
    _fields_ = [("diag_width", ctypes.c_int32), ("band_width", ctypes.c_int32),
                ("frame_tokens", ctypes.c_int32),
                ("reach", ctypes.c_int32), ("stripe_period", ctypes.c_int32),
                ("stripe_width", ctypes.c_int32)]


PATTERN_EMPTY, PATTERN_DIAGONAL, PATTERN_MULTI_DIAGONAL, PATTERN_VERTICAL_STRIPE, PATTERN_DENSE = range(5)

_VP = ctypes.c_void_p
_PP = ctypes.POINTER(Problem)
_SIGS = {
    "tsa_mask_row_words": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32]),
    "tsa_workspace_size": (ctypes.c_int, [ctypes.c_int, _PP, ctypes.POINTER(ctypes.c_size_t)]),
    "tsa_attention_fwd": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP, _VP,
                                         ctypes.c_size_t, _VP]),
    "tsa_attention_fwd_noalloc": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP, _VP]),
    "tsa_attention_bwd": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_float,
                                         _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "tsa_mask_compact": (ctypes.c_int, [_PP, _VP, _VP, _VP, ctypes.c_int64, _VP, ctypes.c_size_t,
                                        _VP]),
    "tsa_predict_mask": (ctypes.c_int, [_PP, _VP, _VP, ctypes.c_int32, _VP, _VP, ctypes.c_size_t,
                                        _VP]),
    "tsa_maskgen_hash": (ctypes.c_int, [_PP, ctypes.POINTER(MaskgenParams), _VP, _VP]),
    "tsa_maskgen_structured": (ctypes.c_int, [_PP, ctypes.POINTER(StructuredParams),
                                              ctypes.POINTER(ctypes.c_int32), _VP, _VP]),
    "tsa_mask_diff": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP]),
    "tsa_quantize_qk_fp8": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "tsa_attention_fwd_fp8": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP,
                                             _VP, ctypes.c_size_t, _VP]),
    "tsa_set_timing_events": (ctypes.c_int, [_VP, _VP]),
    "tsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tsa_last_error": (ctypes.c_char_p, []),
}
EXPORTS = tuple(_SIGS)

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python tile_sparse_attention_amd/build.py`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int):
    if status != OK:
        raise TsaError(status, lib().tsa_last_error().decode())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TsaError(ERR_UNSUPPORTED, f"dtype {t.dtype} (need float32 or bfloat16)")


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise TsaError(ERR_INVALID_ARGUMENT, "tensors must be contiguous GPU tensors")


def problem(B, H, L, d, M, N, dtype=DTYPE_BF16) -> Problem:
    return Problem(B, H, L, d, M, N, dtype)


def mask_row_words(L: int, N: int) -> int:
    return int(lib().tsa_mask_row_words(L, N))


def workspace_size(op: int, pr: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().tsa_workspace_size(op, ctypes.byref(pr), ctypes.byref(n)))
    return int(n.value)


def _workspace(op: int, pr: Problem, device):
    n = workspace_size(op, pr)
    if n == 0:
        return None, 0
    return _torch().empty(n, dtype=_torch().uint8, device=device), n


def _check_fwd_args(q, k, v, mask_bits, M, N, out, lse):
    torch = _torch()
    B, H, L, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or out.shape != q.shape:
        raise TsaError(ERR_INVALID_ARGUMENT, "q, k, v, out must have one shape")
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise TsaError(ERR_INVALID_ARGUMENT, "q, k, v, out must have one dtype")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L)):
        raise TsaError(ERR_INVALID_ARGUMENT, "lse must be float32 [B, H, L]")
    T_q = -(-L // M)
    if mask_bits.dtype not in (torch.int32, torch.uint32) or \
            tuple(mask_bits.shape) != (B, H, T_q, mask_row_words(L, N)):
        raise TsaError(ERR_INVALID_ARGUMENT, "mask_bits must be int32/uint32 [B, H, T_q, words]")


def attention_fwd(q, k, v, mask_bits, M: int, N: int, scale: float | None = None, *,
                  out=None, return_lse: bool = False, workspace=None):
    """O (and optionally LSE) of tile-sparse attention; q, k, v: [B, H, L, d].

    `workspace` (uint8 GPU tensor of at least workspace_size(OP_ATTENTION_FWD)
    bytes) is allocated per call when not given.
    """
    torch = _torch()
    B, H, L, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if return_lse else None
    _need_cuda(q, k, v, mask_bits, out, lse)
    _check_fwd_args(q, k, v, mask_bits, M, N, out, lse)
    pr = Problem(B, H, L, d, M, N, _dtype_code(q))
    if workspace is None:
        ws, nws = _workspace(OP_ATTENTION_FWD, pr, q.device)
    else:
        _need_cuda(workspace)
        ws, nws = workspace, workspace.numel() * workspace.element_size()
    _check(lib().tsa_attention_fwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(mask_bits),
                                   ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(ws), nws,
                                   _stream()))
    return (out, lse) if return_lse else out


def attention_fwd_noalloc(q, k, v, mask_bits, M: int, N: int, scale: float | None = None, *,
                          out, lse=None):
    """tsa_attention_fwd_noalloc: O (and LSE when `lse` is given) written into
    the caller's tensors, with the library's static scratch instead of a
    workspace; the call allocates nothing, so `out` (and `lse`) are required."""
    B, H, L, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need_cuda(q, k, v, mask_bits, out, lse)
    _check_fwd_args(q, k, v, mask_bits, M, N, out, lse)
    pr = Problem(B, H, L, d, M, N, _dtype_code(q))
    _check(lib().tsa_attention_fwd_noalloc(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(mask_bits),
                                           ctypes.c_float(scale), _ptr(out), _ptr(lse), _stream()))
    return (out, lse) if lse is not None else out


def set_timing_events(start=None, stop=None):
    """Record torch.cuda.Event `start` / `stop` around the attention kernels of
    the forward calls that follow (None, None: off)."""
    for e in (start, stop):
        if e is not None and not e.cuda_event:
            e.record()   # torch creates the HIP event on its first record
    _check(lib().tsa_set_timing_events(ctypes.c_void_p(start.cuda_event) if start is not None else None,
                                       ctypes.c_void_p(stop.cuda_event) if stop is not None else None))


def quantize_qk_fp8(q, k):
    """(q8 uint8, q_scale float32 [B, H, ceil(L/16)], k8 uint8, k_scale float32 [B, H])
    of bf16 q, k [B, H, L, 128]: e4m3 bytes with per-tile scales."""
    torch = _torch()
    _need_cuda(q, k)
    B, H, L, d = q.shape
    if k.shape != q.shape or q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise TsaError(ERR_INVALID_ARGUMENT, "q, k must be bf16 of one shape")
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=q.device)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=q.device)
    qs = torch.empty((B, H, -(-L // 16)), dtype=torch.float32, device=q.device)
    ks = torch.empty((B, H), dtype=torch.float32, device=q.device)
    pr = Problem(B, H, L, d, 16, 16, DTYPE_BF16)
    _check(lib().tsa_quantize_qk_fp8(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks),
                                     _stream()))
    return q8, qs, k8, ks


def attention_fwd_fp8(q8, k8, q_scale, k_scale, v, mask_bits, M: int, N: int, scale: float | None = None, *,
                      out=None, return_lse: bool = False, workspace=None):
    """O (and optionally LSE) of tile-sparse attention with FP8 scores: q8, k8
    and the scales as quantize_qk_fp8 returns them, v bf16 [B, H, L, 128]."""
    torch = _torch()
    B, H, L, d = v.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(v)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=v.device) if return_lse else None
    _need_cuda(q8, k8, q_scale, k_scale, v, mask_bits, out, lse)
    if q8.shape != v.shape or k8.shape != v.shape or q8.dtype != torch.uint8 or k8.dtype != torch.uint8:
        raise TsaError(ERR_INVALID_ARGUMENT, "q8, k8 must be uint8 of v's shape")
    if tuple(q_scale.shape) != (B, H, -(-L // 16)) or tuple(k_scale.shape) != (B, H):
        raise TsaError(ERR_INVALID_ARGUMENT, "q_scale [B, H, ceil(L/16)], k_scale [B, H] float32")
    T_q = -(-L // M)
    if mask_bits.dtype not in (torch.int32, torch.uint32) or \
            tuple(mask_bits.shape) != (B, H, T_q, mask_row_words(L, N)):
        raise TsaError(ERR_INVALID_ARGUMENT, "mask_bits must be int32/uint32 [B, H, T_q, words]")
    pr = Problem(B, H, L, d, M, N, DTYPE_BF16)
    if workspace is None:
        ws, nws = _workspace(OP_ATTENTION_FWD, pr, v.device)
    else:
        _need_cuda(workspace)
        ws, nws = workspace, workspace.numel() * workspace.element_size()
    _check(lib().tsa_attention_fwd_fp8(ctypes.byref(pr), _ptr(q8), _ptr(k8), _ptr(q_scale), _ptr(k_scale),
                                       _ptr(v), _ptr(mask_bits), ctypes.c_float(scale), _ptr(out), _ptr(lse),
                                       _ptr(ws), nws, _stream()))
    return (out, lse) if return_lse else out


def attention_bwd(q, k, v, o, do, lse, mask_bits, M: int, N: int, scale: float | None = None, *,
                  workspace=None):
    """(dQ, dK, dV) of tile-sparse attention for the upstream gradient `do`.

    q, k, v, o, do: bf16 [B, H, L, d] (o and lse as the forward returned them
    with return_lse=True).  `workspace` (uint8 GPU tensor of at least
    workspace_size(OP_ATTENTION_BWD) bytes) is allocated per call when not given.
    """
    torch = _torch()
    B, H, L, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need_cuda(q, k, v, o, do, lse, mask_bits)
    for t in (k, v, o, do):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise TsaError(ERR_INVALID_ARGUMENT, "q, k, v, o, do must have one shape and dtype")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L):
        raise TsaError(ERR_INVALID_ARGUMENT, "lse must be float32 [B, H, L]")
    T_q = -(-L // M)
    if mask_bits.dtype not in (torch.int32, torch.uint32) or \
            tuple(mask_bits.shape) != (B, H, T_q, mask_row_words(L, N)):
        raise TsaError(ERR_INVALID_ARGUMENT, "mask_bits must be int32/uint32 [B, H, T_q, words]")
    pr = Problem(B, H, L, d, M, N, _dtype_code(q))
    if workspace is None:
        ws, nws = _workspace(OP_ATTENTION_BWD, pr, q.device)
    else:
        _need_cuda(workspace)
        ws, nws = workspace, workspace.numel() * workspace.element_size()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    _check(lib().tsa_attention_bwd(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                                   _ptr(lse), _ptr(mask_bits), ctypes.c_float(scale), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(ws), nws, _stream()))
    return dq, dk, dv


def mask_diff(mask_a, mask_b, L: int, M: int, N: int):
    """(row_changed int64 [B, H, T_q], head_changed int64 [B, H]): per bitmap row
    and per head, the number of key tiles whose keep bit differs between two
    masks [B, H, T_q, words] of one problem."""
    torch = _torch()
    _need_cuda(mask_a, mask_b)
    B, H, T_q, words = mask_a.shape
    if tuple(mask_b.shape) != tuple(mask_a.shape) or words != mask_row_words(L, N) or T_q != -(-L // M):
        raise TsaError(ERR_INVALID_ARGUMENT, "masks must both be [B, H, T_q, words] of the problem")
    for m in (mask_a, mask_b):
        if m.dtype not in (torch.int32, torch.uint32):
            raise TsaError(ERR_INVALID_ARGUMENT, "masks must be int32/uint32")
    rows = torch.empty((B, H, T_q), dtype=torch.int64, device=mask_a.device)
    heads = torch.empty((B, H), dtype=torch.int64, device=mask_a.device)
    pr = Problem(B, H, L, 0, M, N, DTYPE_BF16)
    _check(lib().tsa_mask_diff(ctypes.byref(pr), _ptr(mask_a), _ptr(mask_b), _ptr(rows), _ptr(heads),
                               _stream()))
    return rows, heads


def mask_compact(mask_bits, L: int, M: int, N: int, col_capacity: int | None = None):
    """(row_ptr int64 [rows+1], col_idx int32) of a bitmap [B, H, T_q, words].

    With col_capacity None the list length is read back from a first pass
    (one host synchronisation) and col_idx is sized exactly.
    """
    torch = _torch()
    B, H, T_q, words = mask_bits.shape
    _need_cuda(mask_bits)
    pr = Problem(B, H, L, 0, M, N, DTYPE_BF16)
    if T_q != -(-L // M) or words != mask_row_words(L, N):
        raise TsaError(ERR_INVALID_ARGUMENT, "mask_bits shape does not match L, M, N")
    ws, nws = _workspace(OP_MASK_COMPACT, pr, mask_bits.device)
    rows = B * H * T_q
    row_ptr = torch.empty(rows + 1, dtype=torch.int64, device=mask_bits.device)
    if col_capacity is None:
        _check(lib().tsa_mask_compact(ctypes.byref(pr), _ptr(mask_bits), _ptr(row_ptr),
                                      ctypes.c_void_p(0), 0, _ptr(ws), nws, _stream()))
        col_capacity = int(row_ptr[-1].item())
    col_idx = torch.empty(max(col_capacity, 1), dtype=torch.int32, device=mask_bits.device)
    _check(lib().tsa_mask_compact(ctypes.byref(pr), _ptr(mask_bits), _ptr(row_ptr), _ptr(col_idx),
                                  col_capacity, _ptr(ws), nws, _stream()))
    return row_ptr, col_idx[:col_capacity]


def predict_mask(q, k, M: int, N: int, sparsity_percent: int = 85, *, out=None):
    """Predicted keep-bitmap [B, H, T_q, words] (int32 storage of uint32 words)."""
    torch = _torch()
    B, H, L, d = q.shape
    _need_cuda(q, k)
    if k.shape != q.shape or k.dtype != q.dtype:
        raise TsaError(ERR_INVALID_ARGUMENT, "q and k must have one shape and dtype")
    pr = Problem(B, H, L, d, M, N, _dtype_code(q))
    T_q = -(-L // M)
    if out is None:
        out = torch.empty((B, H, T_q, mask_row_words(L, N)), dtype=torch.int32, device=q.device)
    _need_cuda(out)
    ws, nws = _workspace(OP_PREDICT_MASK, pr, q.device)
    _check(lib().tsa_predict_mask(ctypes.byref(pr), _ptr(q), _ptr(k), int(sparsity_percent),
                                  _ptr(out), _ptr(ws), nws, _stream()))
    return out


def maskgen_hash(B, H, L, M, N, *, state0: int, thr_near: int, thr_far: int,
                 frame_tokens: int = 0, frame_radius: int = 0, force_diag: bool = True,
                 device="cuda"):
    """Synthetic keep-bitmap from the counter-based generator of tsa_workload.h."""
    torch = _torch()
    pr = Problem(B, H, L, 0, M, N, DTYPE_BF16)
    out = torch.empty((B, H, -(-L // M), mask_row_words(L, N)), dtype=torch.int32, device=device)
    g = MaskgenParams(state0 & 0xFFFFFFFFFFFFFFFF, thr_near, thr_far, frame_tokens, frame_radius,
                      1 if force_diag else 0)
    _check(lib().tsa_maskgen_hash(ctypes.byref(pr), ctypes.byref(g), _ptr(out), _stream()))
    return out


def maskgen_structured(B, H, L, M, N, head_patterns, *, diag_width: int = 0, band_width: int = 0,
                       frame_tokens: int = 0, reach: int = 0, stripe_period: int = 0,
                       stripe_width: int = 0, device="cuda"):
    """Structured keep-bitmap (tsa_workload.h): one PATTERN_* per head."""
    torch = _torch()
    if len(head_patterns) != H:
        raise TsaError(ERR_INVALID_ARGUMENT, "one pattern per head")
    pr = Problem(B, H, L, 0, M, N, DTYPE_BF16)
    out = torch.empty((B, H, -(-L // M), mask_row_words(L, N)), dtype=torch.int32, device=device)
    g = StructuredParams(diag_width, band_width, frame_tokens, reach, stripe_period, stripe_width)
    pats = (ctypes.c_int32 * H)(*[int(x) for x in head_patterns])
    _check(lib().tsa_maskgen_structured(ctypes.byref(pr), ctypes.byref(g), pats, _ptr(out),
                                        _stream()))
    return out


def status_string(status: int) -> str:
    return lib().tsa_status_string(status).decode()


def last_error() -> str:
    return lib().tsa_last_error().decode()
