"""ctypes binding of libbsa.so (C ABI in include/bsa.h).

Argument marshalling only: tensors are described by pointer, dtype and
strides, outputs are allocated with torch on the caller's device, and every
computation happens in the HIP kernels behind the C entry points.  Importing
this module does not need a GPU; calling an entry point without the built
library raises immediately.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# BSA_LIBRARY selects another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("BSA_LIBRARY") or os.path.join(_PKG, "libbsa.so")

BSA_OK, BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED, BSA_ERR_WORKSPACE, BSA_ERR_HIP = range(5)
BSA_BF16, BSA_F32 = 0, 1
BSA_PAT_DENSE, BSA_PAT_BLOCK, BSA_PAT_VS = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 16 << 20   # BSA_NOALLOC_SCRATCH_BYTES of include/bsa.h
GATE_SKIPPED = {"drop": 0, "count": 1}   # bsa_gate_skipped

EXPORTS = ("bsa_status_string", "bsa_workspace_size", "bsa_fwd", "bsa_fwd_partials", "bsa_num_partials",
           "bsa_speculative_sparse", "bsa_speculative_sparse_noalloc", "bsa_speculative_partials", "bsa_speculative_num_partials",
           "bsa_speculative_workspace_size", "bsa_combine", "bsa_fwd_gated", "bsfa_calibrate",
           "bsa_selected_workspace_size", "bsa_fwd_selected", "bsa_bwd_workspace_size", "bsa_bwd",
           "vs_convert_indexes", "vs_convert_indexes_mergehead", "bsa_check_pattern")


class BSAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class _Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("Sq", ctypes.c_int32),
                ("Sk", ctypes.c_int32), ("D", ctypes.c_int32), ("cu_seqlens_q", ctypes.c_void_p),
                ("cu_seqlens_k", ctypes.c_void_p), ("max_seqlen_q", ctypes.c_int32),
                ("max_seqlen_k", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("softcap", ctypes.c_float)]


class _Pattern(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("Ht", ctypes.c_int32), ("block_M", ctypes.c_int32),
                ("block_N", ctypes.c_int32), ("cap", ctypes.c_int32), ("col_cap", ctypes.c_int32),
                ("count", ctypes.c_void_p), ("index", ctypes.c_void_p), ("col_count", ctypes.c_void_p),
                ("col_index", ctypes.c_void_p), ("s_b", ctypes.c_int64), ("s_h", ctypes.c_int64),
                ("s_q", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libbsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m long_context_attention_sparse_amd.build`")
    lib = ctypes.CDLL(path)
    lib.bsa_status_string.restype = ctypes.c_char_p
    lib.bsa_status_string.argtypes = [ctypes.c_int]
    lib.bsa_workspace_size.restype = ctypes.c_size_t
    lib.bsa_workspace_size.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Pattern)]
    lib.bsa_fwd.restype = ctypes.c_int
    lib.bsa_fwd.argtypes = [ctypes.POINTER(_Problem), _Tensor, _Tensor, _Tensor, ctypes.POINTER(_Pattern), _Tensor,
                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.bsa_fwd_partials.restype = ctypes.c_int
    lib.bsa_fwd_partials.argtypes = [ctypes.POINTER(_Problem), _Tensor, _Tensor, _Tensor, ctypes.POINTER(_Pattern),
                                     ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.bsa_num_partials.restype = ctypes.c_int32
    lib.bsa_num_partials.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Pattern), ctypes.c_int32]
    spec_args = [ctypes.POINTER(_Problem), _Tensor, _Tensor, _Tensor, ctypes.c_int32, ctypes.c_int32, _Tensor,
                 _Tensor, ctypes.POINTER(_Pattern)]
    lib.bsa_speculative_sparse.restype = ctypes.c_int
    lib.bsa_speculative_sparse.argtypes = spec_args + [_Tensor, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                                       ctypes.c_void_p]
    lib.bsa_speculative_sparse_noalloc.restype = ctypes.c_int
    lib.bsa_speculative_sparse_noalloc.argtypes = spec_args + [_Tensor, ctypes.c_void_p, ctypes.c_void_p]
    lib.bsa_speculative_partials.restype = ctypes.c_int
    lib.bsa_speculative_partials.argtypes = spec_args + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.bsa_speculative_num_partials.restype = ctypes.c_int32
    lib.bsa_speculative_num_partials.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32, ctypes.POINTER(_Pattern)]
    lib.bsa_speculative_workspace_size.restype = ctypes.c_size_t
    lib.bsa_speculative_workspace_size.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32,
                                                   ctypes.POINTER(_Pattern)]
    lib.bsa_combine.restype = ctypes.c_int
    lib.bsa_combine.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_void_p, ctypes.c_void_p, _Tensor, ctypes.c_void_p,
                                                      ctypes.c_void_p]
    lib.bsa_fwd_gated.restype = ctypes.c_int
    lib.bsa_fwd_gated.argtypes = [ctypes.POINTER(_Problem), _Tensor, _Tensor, _Tensor, ctypes.c_void_p,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _Tensor, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.bsa_selected_workspace_size.restype = ctypes.c_size_t
    lib.bsa_selected_workspace_size.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32]
    lib.bsa_fwd_selected.restype = ctypes.c_int
    lib.bsa_fwd_selected.argtypes = [ctypes.POINTER(_Problem), _Tensor, _Tensor, _Tensor, ctypes.c_void_p,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _Tensor, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.bsa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.bsa_bwd_workspace_size.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Pattern)]
    lib.bsa_bwd.restype = ctypes.c_int
    lib.bsa_bwd.argtypes = [ctypes.POINTER(_Problem), _Tensor, _Tensor, _Tensor, ctypes.POINTER(_Pattern), _Tensor,
                            ctypes.c_void_p, _Tensor, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.bsfa_calibrate.restype = ctypes.c_int
    lib.bsfa_calibrate.argtypes = [ctypes.POINTER(_Problem), _Tensor, _Tensor, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.vs_convert_indexes.restype = ctypes.c_int
    lib.vs_convert_indexes.argtypes = ([ctypes.c_void_p] * 4 + [ctypes.c_int32] * 8 + [ctypes.c_void_p] * 5)
    lib.vs_convert_indexes_mergehead.restype = ctypes.c_int
    lib.vs_convert_indexes_mergehead.argtypes = ([ctypes.c_void_p] * 6 + [ctypes.c_int32] * 8 +
                                                 [ctypes.c_void_p] * 5)
    lib.bsa_check_pattern.restype = ctypes.c_int
    lib.bsa_check_pattern.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Pattern), ctypes.c_void_p,
                                      ctypes.c_void_p]
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != BSA_OK:
        raise BSAError(fn, status, load().bsa_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tensor(t: torch.Tensor, varlen: bool = False) -> _Tensor:
    """[B, S, H, D] (or varlen [T, H, D]) view with a contiguous last axis."""
    if t.stride(-1) != 1:
        raise ValueError("the head-dim axis must be contiguous")
    if varlen:
        if t.dim() != 3:
            raise ValueError("varlen tensors are [total, heads, head_dim]")
        return _Tensor(t.data_ptr(), _dtype_code(t), 0, t.stride(0), t.stride(1))
    if t.dim() != 4:
        raise ValueError("tensors are [batch, seq, heads, head_dim]")
    return _Tensor(t.data_ptr(), _dtype_code(t), t.stride(0), t.stride(1), t.stride(2))


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 device tensor")
    return t


@dataclass
class BlockPattern:
    """Per-query-block lists of key-block ids.

    count [B, Ht, nQB] and index [B, Ht, nQB, cap] (int32, device).  Ht is Hq
    or Hkv.  A 1-D table of N ids shared by every row and head (the form of the
    sparse block-table forward) is ``BlockPattern.table(ids, block_size)``.
    """
    count: torch.Tensor
    index: torch.Tensor
    block_M: int
    block_N: int
    broadcast: bool = False

    @staticmethod
    def table(ids: torch.Tensor, block_size: int, block_M: int = 128) -> "BlockPattern":
        ids = _i32(ids.reshape(-1), "table")
        count = torch.tensor([ids.numel()], dtype=torch.int32, device=ids.device)
        return BlockPattern(count, ids, block_M, block_size, broadcast=True)

    def struct(self, Hq: int) -> _Pattern:
        _i32(self.count, "count")
        _i32(self.index, "index")
        if self.broadcast:
            return _Pattern(BSA_PAT_BLOCK, Hq, self.block_M, self.block_N, self.index.numel(), 0,
                            self.count.data_ptr(), self.index.data_ptr(), None, None, 0, 0, 0)
        B, Ht, nqb = self.count.shape
        cap = self.index.shape[-1]
        if tuple(self.index.shape[:3]) != (B, Ht, nqb):
            raise ValueError("index must be [B, Ht, nQB, cap] matching count")
        return _Pattern(BSA_PAT_BLOCK, Ht, self.block_M, self.block_N, cap, 0, self.count.data_ptr(),
                        self.index.data_ptr(), None, None, Ht * nqb, nqb, 1)


@dataclass
class VSPattern:
    """Converted vertical-slash metadata: block_count [B,H,R], block_offset [B,H,R,NNZ_S],
    column_count [B,H,R], column_index [B,H,R,NNZ_V] (int32, device)."""
    block_count: torch.Tensor
    block_offset: torch.Tensor
    column_count: torch.Tensor
    column_index: torch.Tensor
    block_M: int = 64
    block_N: int = 64

    def struct(self, Hq: int) -> _Pattern:
        B, H, R = self.block_count.shape
        for n, t in (("block_count", self.block_count), ("block_offset", self.block_offset),
                     ("column_count", self.column_count), ("column_index", self.column_index)):
            _i32(t, n)
        return _Pattern(BSA_PAT_VS, H, self.block_M, self.block_N, self.block_offset.shape[-1],
                        self.column_index.shape[-1], self.block_count.data_ptr(), self.block_offset.data_ptr(),
                        self.column_count.data_ptr(), self.column_index.data_ptr(), H * R, R, 1)


def _problem(q, k, causal, softmax_scale, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=0, max_seqlen_k=0,
             softcap=0.0):
    if cu_seqlens_q is not None:
        B = cu_seqlens_q.numel() - 1
        _, Hq, D = q.shape
        Hkv = k.shape[1]
        return _Problem(B, Hq, Hkv, int(max_seqlen_q), int(max_seqlen_k), D,
                        _i32(cu_seqlens_q, "cu_seqlens_q").data_ptr(), _i32(cu_seqlens_k, "cu_seqlens_k").data_ptr(),
                        int(max_seqlen_q), int(max_seqlen_k), float(softmax_scale or 0.0), int(bool(causal)),
                        float(softcap or 0.0))
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    return _Problem(B, Hq, Hkv, Sq, Sk, D, None, None, 0, 0, float(softmax_scale or 0.0), int(bool(causal)),
                    float(softcap or 0.0))


def bsa_workspace_size(q, k, pattern=None, causal=False, **varlen) -> int:
    prob = _problem(q, k, causal, None, **varlen)
    pat = pattern.struct(prob.Hq) if pattern is not None else None
    return int(load().bsa_workspace_size(ctypes.byref(prob), ctypes.byref(pat) if pat is not None else None))


def bsa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pattern=None, *, causal: bool = False,
            softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            out_dtype: torch.dtype = torch.bfloat16, lse: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, cu_seqlens_q=None, cu_seqlens_k=None,
            max_seqlen_q: int = 0, max_seqlen_k: int = 0, softcap: float = 0.0, stream=None):
    """Attention over a key pattern (None = dense).  Returns (out, lse).

    q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D] bf16 (or varlen [total, H, D] with
    cu_seqlens).  out defaults to a new ``out_dtype`` tensor shaped like q;
    lse is float32 [B, Hq, Sq] (varlen: [Hq, total_q]).  softcap > 0 caps every scaled score x
    at softcap * tanh(x / softcap).
    """
    lib = load()
    varlen = cu_seqlens_q is not None
    prob = _problem(q, k, causal, softmax_scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softcap)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse_shape = (q.shape[1], q.shape[0]) if varlen else (q.shape[0], q.shape[2], q.shape[1])
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    pat = pattern.struct(prob.Hq) if pattern is not None else None
    pat_p = ctypes.byref(pat) if pat is not None else None
    need = int(lib.bsa_workspace_size(ctypes.byref(prob), pat_p))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.bsa_fwd(ctypes.byref(prob), _tensor(q, varlen), _tensor(k, varlen), _tensor(v, varlen), pat_p,
                     _tensor(out, varlen), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))
    _check("bsa_fwd", st)
    return out, lse


def bsa_check_pattern(q, k, pattern, *, causal: bool = False, cu_seqlens_q=None, cu_seqlens_k=None,
                      max_seqlen_q: int = 0, max_seqlen_k: int = 0, result: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Checks a BlockPattern or VSPattern on the device against the rules the attention kernels
    assume (ids in range and distinct; VS windows ascending and disjoint, columns ascending and
    outside the windows).  Returns int32 [2] on the device: (violating lists, first violating
    flat list index (b * Ht + h) * nQB + m, or 2**31 - 1 when there is none)."""
    prob = _problem(q, k, causal, None, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    pat = pattern.struct(prob.Hq)
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=q.device)
    _i32(result, "result")
    _check("bsa_check_pattern", load().bsa_check_pattern(ctypes.byref(prob), ctypes.byref(pat), _ptr(result),
                                                         _stream(stream)))
    return result


def bsa_num_partials(q, k, pattern=None, entries_per_partial: int = 1, causal: bool = False) -> int:
    prob = _problem(q, k, causal, None)
    pat = pattern.struct(prob.Hq) if pattern is not None else None
    n = int(load().bsa_num_partials(ctypes.byref(prob), ctypes.byref(pat) if pat is not None else None,
                                    int(entries_per_partial)))
    if n < 0:
        raise BSAError("bsa_num_partials", BSA_ERR_INVALID_ARG, "invalid arguments")
    return n


def bsa_fwd_partials(q, k, v, pattern=None, entries_per_partial: int = 1, *, causal: bool = False,
                     softmax_scale=None, o_part: Optional[torch.Tensor] = None,
                     lse_part: Optional[torch.Tensor] = None, softcap: float = 0.0, stream=None):
    """(o, lse) partials over groups of ``entries_per_partial`` pattern entries (1 = one per
    list entry; a dense pattern's entries are 64-key blocks).  Returns
    o_part [P, B, Sq, Hq, D] and lse_part [P, B, Hq, Sq] (float32); given buffers (views into a
    larger partial buffer, for instance) are filled in place."""
    lib = load()
    prob = _problem(q, k, causal, softmax_scale, softcap=softcap)
    pat = pattern.struct(prob.Hq) if pattern is not None else None
    pat_p = ctypes.byref(pat) if pat is not None else None
    P = int(lib.bsa_num_partials(ctypes.byref(prob), pat_p, int(entries_per_partial)))
    if P < 0:
        raise BSAError("bsa_fwd_partials", BSA_ERR_INVALID_ARG, "invalid arguments")
    B, Sq, Hq, D = q.shape
    if o_part is None:
        o_part = torch.empty((P, B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((P, B, Hq, Sq), dtype=torch.float32, device=q.device)
    if tuple(o_part.shape) != (P, B, Sq, Hq, D) or tuple(lse_part.shape) != (P, B, Hq, Sq):
        raise ValueError(f"partial buffers must be [{P}, B, Sq, Hq, D] and [{P}, B, Hq, Sq]")
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("partial buffers must be contiguous")
    st = lib.bsa_fwd_partials(ctypes.byref(prob), _tensor(q), _tensor(k), _tensor(v), pat_p,
                              int(entries_per_partial), _ptr(o_part), _ptr(lse_part), _stream(stream))
    _check("bsa_fwd_partials", st)
    return o_part, lse_part


def bsa_combine(o_part: torch.Tensor, lse_part: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.bfloat16, lse: Optional[torch.Tensor] = None, stream=None):
    """Log-sum-exp combine of partials o_part [P, B, Sq, Hq, D], lse_part [P, B, Hq, Sq] (float32)."""
    lib = load()
    P, B, Sq, Hq, D = o_part.shape
    if not (o_part.is_contiguous() and lse_part.is_contiguous()) or o_part.dtype != torch.float32:
        raise ValueError("partials must be contiguous float32")
    if tuple(lse_part.shape) != (P, B, Hq, Sq):
        raise ValueError("lse_part must be [P, B, Hq, Sq]")
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=out_dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=o_part.device)
    st = lib.bsa_combine(P, B, Hq, Sq, D, _ptr(o_part), _ptr(lse_part), _tensor(out), _ptr(lse), _stream(stream))
    _check("bsa_combine", st)
    return out, lse


def bsa_fwd_gated(q, k, v, T: torch.Tensor, *, block_M: int = 128, block_N: int = 128, softmax_scale=None,
                  skipped: str = "drop", out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                  return_mask: bool = True, return_tile_max: bool = False, stream=None):
    """BSFA gated causal attention.  ``skipped``: "drop" (a skipped tile's scores are left out of
    the softmax) or "count" (they stay in the maximum and normaliser; only V and P V are skipped).
    Returns (out, lse, keep_mask or None, tile_max or None)."""
    if skipped not in GATE_SKIPPED:
        raise ValueError(f"skipped must be one of {sorted(GATE_SKIPPED)}")
    lib = load()
    prob = _problem(q, k, True, softmax_scale)
    B, S, Hq, D = q.shape
    nqb = S // block_M
    nkb = k.shape[1] // block_N
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    keep = torch.zeros((B, Hq, nqb, nkb), dtype=torch.uint8, device=q.device) if return_mask else None
    tmax = torch.full((B, Hq, nqb, nkb), float("nan"), dtype=torch.float32, device=q.device) \
        if return_tile_max else None
    if T.dim() == 2:  # calibrated [Hq, nQB], shared by the batch
        T = T.unsqueeze(0).expand(B, -1, -1).contiguous()
    if T.dtype != torch.float32 or not T.is_contiguous():
        raise ValueError("T must be contiguous float32 [B, Hq, nQB] (or [Hq, nQB])")
    st = lib.bsa_fwd_gated(ctypes.byref(prob), _tensor(q), _tensor(k), _tensor(v), _ptr(T), block_M, block_N,
                           GATE_SKIPPED[skipped], _tensor(out), _ptr(lse), _ptr(keep), _ptr(tmax), _stream(stream))
    _check("bsa_fwd_gated", st)
    return out, lse, keep, tmax


def bsa_bwd(q, k, v, out, lse, dout, pattern=None, *, causal: bool = False, softmax_scale=None,
            workspace: Optional[torch.Tensor] = None, cu_seqlens_q=None, cu_seqlens_k=None,
            max_seqlen_q: int = 0, max_seqlen_k: int = 0, softcap: float = 0.0, stream=None):
    """Gradients of bsa_fwd(q, k, v, pattern, causal=...) given its (out, lse) and the upstream
    gradient dout (and the same softcap).  Returns dq shaped like q, dk and dv shaped like k
    (float32): [B, S, H, D], or packed [total, H, D] with cu_seqlens (lse then [Hq, total_q], as
    bsa_fwd returns it)."""
    lib = load()
    varlen = cu_seqlens_q is not None
    prob = _problem(q, k, causal, softmax_scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softcap)
    pat = pattern.struct(prob.Hq) if pattern is not None else None
    pat_p = ctypes.byref(pat) if pat is not None else None
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 ([B, Hq, Sq], or [Hq, total_q] with cu_seqlens)")
    need = int(lib.bsa_bwd_workspace_size(ctypes.byref(prob), pat_p))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.bsa_bwd(ctypes.byref(prob), _tensor(q, varlen), _tensor(k, varlen), _tensor(v, varlen), pat_p,
                     _tensor(out, varlen), _ptr(lse), _tensor(dout, varlen), _ptr(dq), _ptr(dk), _ptr(dv),
                     _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("bsa_bwd", st)
    return dq, dk, dv


def bsa_bwd_workspace_size(q, k, pattern=None, causal: bool = False) -> int:
    prob = _problem(q, k, causal, None)
    pat = pattern.struct(prob.Hq) if pattern is not None else None
    return int(load().bsa_bwd_workspace_size(ctypes.byref(prob), ctypes.byref(pat) if pat is not None else None))


def bsa_fwd_selected(q, k, v, sel: torch.Tensor, *, block_size: int = 64, causal: bool = True,
                     softmax_scale=None, softcap: float = 0.0, out: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.bfloat16, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, cu_seqlens_q=None, cu_seqlens_k=None,
                     max_seqlen_q: int = 0, max_seqlen_k: int = 0, stream=None):
    """Selected attention: each query token attends to the key blocks it selected.
    sel int32 [B, Sq, Hkv, topk] (varlen: [total_q, Hkv, topk]), -1 = unused slot.
    Returns (out, lse) as bsa_fwd."""
    lib = load()
    varlen = cu_seqlens_q is not None
    prob = _problem(q, k, causal, softmax_scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softcap)
    sel = _i32(sel, "sel")
    topk = sel.shape[-1]
    total_q = q.shape[0] if varlen else 0
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        shape = (q.shape[1], q.shape[0]) if varlen else (q.shape[0], q.shape[2], q.shape[1])
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    need = int(lib.bsa_selected_workspace_size(ctypes.byref(prob), total_q, topk, block_size))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.bsa_fwd_selected(ctypes.byref(prob), _tensor(q, varlen), _tensor(k, varlen), _tensor(v, varlen),
                              _ptr(sel), total_q, topk, block_size, _tensor(out, varlen), _ptr(lse), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check("bsa_fwd_selected", st)
    return out, lse


def bsa_selected_workspace_size(q, k, topk: int, *, block_size: int = 64, cu_seqlens_q=None, cu_seqlens_k=None,
                                max_seqlen_q: int = 0, max_seqlen_k: int = 0) -> int:
    prob = _problem(q, k, True, None, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    total_q = q.shape[0] if cu_seqlens_q is not None else 0
    return int(load().bsa_selected_workspace_size(ctypes.byref(prob), total_q, int(topk), int(block_size)))


def bsfa_calibrate(q, k, k_keep: int, *, softmax_scale=None, tile_max: Optional[torch.Tensor] = None,
                   stream=None):
    """BSFA threshold calibration over calibration samples q [B, S, Hq, D], k [B, S, Hkv, D]:
    per (b, head, 128-row query block i) the k_keep-th largest off-diagonal tile maximum, -inf
    for i < k_keep, averaged over the samples.  Returns (T [Hq, nQB], tile_max [B, Hq, nQB, nQB])
    (float32; tile_max entries above the diagonal are left as given, NaN when allocated here)."""
    lib = load()
    prob = _problem(q, k, True, softmax_scale)
    B, S, Hq, D = q.shape
    nqb = S // 128
    if tile_max is None:
        tile_max = torch.full((B, Hq, nqb, nqb), float("nan"), dtype=torch.float32, device=q.device)
    if tile_max.dtype != torch.float32 or not tile_max.is_contiguous() or tile_max.numel() != B * Hq * nqb * nqb:
        raise ValueError("tile_max must be contiguous float32 [B, Hq, nQB, nQB]")
    T = torch.empty((Hq, nqb), dtype=torch.float32, device=q.device)
    st = lib.bsfa_calibrate(ctypes.byref(prob), _tensor(q), _tensor(k), int(k_keep), _ptr(tile_max), _ptr(T),
                            _stream(stream))
    _check("bsfa_calibrate", st)
    return T, tile_max


def _vs_outputs(vertical_indexes, slash_indexes, context_size, block_size_M):
    B, H, nnz_v = vertical_indexes.shape
    nnz_s = slash_indexes.shape[-1]
    rows = (context_size + block_size_M - 1) // block_size_M
    dev = vertical_indexes.device
    return (torch.empty((B, H, rows), dtype=torch.int32, device=dev),
            torch.empty((B, H, rows, nnz_s), dtype=torch.int32, device=dev),
            torch.empty((B, H, rows), dtype=torch.int32, device=dev),
            torch.empty((B, H, rows, nnz_v), dtype=torch.int32, device=dev))


def vs_convert_indexes(q_seqlens, kv_seqlens, vertical_indexes, slash_indexes, context_size: int,
                       block_size_M: int = 64, block_size_N: int = 64, causal: bool = True, stream=None):
    """Vertical-slash conversion.  Returns (block_count, block_offset, column_count, column_index)."""
    lib = load()
    B, H, nnz_v = vertical_indexes.shape
    nnz_s = slash_indexes.shape[-1]
    bc, bo, cc, ci = _vs_outputs(vertical_indexes, slash_indexes, context_size, block_size_M)
    st = lib.vs_convert_indexes(_ptr(_i32(q_seqlens, "q_seqlens")), _ptr(_i32(kv_seqlens, "kv_seqlens")),
                                _ptr(_i32(vertical_indexes, "vertical_indexes")),
                                _ptr(_i32(slash_indexes, "slash_indexes")), B, H, nnz_v, nnz_s, int(context_size),
                                int(block_size_M), int(block_size_N), int(bool(causal)), _ptr(bc), _ptr(bo),
                                _ptr(cc), _ptr(ci), _stream(stream))
    _check("vs_convert_indexes", st)
    return bc, bo, cc, ci


def vs_convert_indexes_mergehead(q_seqlens, kv_seqlens, vertical_indexes, slash_indexes, vertical_indices_count,
                                 slash_indices_count, context_size: int, block_size_M: int = 64,
                                 block_size_N: int = 64, causal: bool = True, stream=None):
    """Vertical-slash conversion with per-head counts (int32 [H]) of valid indices.
    Returns (block_count, block_offset, column_count, column_index)."""
    lib = load()
    B, H, nnz_v = vertical_indexes.shape
    nnz_s = slash_indexes.shape[-1]
    vc = _i32(vertical_indices_count, "vertical_indices_count")
    sc = _i32(slash_indices_count, "slash_indices_count")
    if vc.numel() != H or sc.numel() != H:
        raise ValueError("vertical_indices_count and slash_indices_count need one entry per head")
    bc, bo, cc, ci = _vs_outputs(vertical_indexes, slash_indexes, context_size, block_size_M)
    st = lib.vs_convert_indexes_mergehead(_ptr(_i32(q_seqlens, "q_seqlens")), _ptr(_i32(kv_seqlens, "kv_seqlens")),
                                          _ptr(_i32(vertical_indexes, "vertical_indexes")),
                                          _ptr(_i32(slash_indexes, "slash_indexes")), _ptr(vc), _ptr(sc), B, H,
                                          nnz_v, nnz_s, int(context_size), int(block_size_M), int(block_size_N),
                                          int(bool(causal)), _ptr(bc), _ptr(bo), _ptr(cc), _ptr(ci),
                                          _stream(stream))
    _check("vs_convert_indexes_mergehead", st)
    return bc, bo, cc, ci


def bsa_speculative_partials(q, k_spec, v_spec, k, v, missed: BlockPattern, *, causal_spec: bool = True,
                             softmax_scale=None, o_part: Optional[torch.Tensor] = None,
                             lse_part: Optional[torch.Tensor] = None, softcap: float = 0.0, stream=None):
    """Partials of both passes of speculative + sparse decoding (one launch on the decode path).
    Returns o_part [P, B, Sq, Hq, D], lse_part [P, B, Hq, Sq] (float32)."""
    lib = load()
    prob = _problem(q, k, False, softmax_scale, softcap=softcap)
    pat = missed.struct(prob.Hq)
    Sk_spec = k_spec.shape[1]
    P = int(lib.bsa_speculative_num_partials(ctypes.byref(prob), Sk_spec, ctypes.byref(pat)))
    if P < 0:
        raise BSAError("bsa_speculative_partials", BSA_ERR_INVALID_ARG, "invalid arguments")
    B, Sq, Hq, D = q.shape
    if o_part is None:
        o_part = torch.empty((P, B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((P, B, Hq, Sq), dtype=torch.float32, device=q.device)
    if tuple(o_part.shape) != (P, B, Sq, Hq, D) or tuple(lse_part.shape) != (P, B, Hq, Sq):
        raise ValueError(f"partial buffers must be [{P}, B, Sq, Hq, D] and [{P}, B, Hq, Sq]")
    st = lib.bsa_speculative_partials(ctypes.byref(prob), _tensor(q), _tensor(k_spec), _tensor(v_spec), Sk_spec,
                                      int(bool(causal_spec)), _tensor(k), _tensor(v), ctypes.byref(pat),
                                      _ptr(o_part), _ptr(lse_part), _stream(stream))
    _check("bsa_speculative_partials", st)
    return o_part, lse_part


def speculative_sparse(q, k_spec, v_spec, k, v, missed: BlockPattern, *, causal_spec: bool = True,
                       softmax_scale=None, out_dtype: torch.dtype = torch.bfloat16, out=None, lse=None,
                       workspace=None, softcap: float = 0.0, stream=None):
    """Speculative + sparse decoding with exact combine ("Sparse FlashAttention with
    Incremental Repair", Usage 2): attention over (k_spec, v_spec) with the causal flag
    (the speculative pass), attention over the missed blocks of (k, v) without a mask (the
    repair pass), and the log-sum-exp combine.  Returns (out, lse)."""
    lib = load()
    prob = _problem(q, k, False, softmax_scale, softcap=softcap)
    pat = missed.struct(prob.Hq)
    Sk_spec = k_spec.shape[1]
    B, Sq, Hq, D = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    need = int(lib.bsa_speculative_workspace_size(ctypes.byref(prob), Sk_spec, ctypes.byref(pat)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib.bsa_speculative_sparse(ctypes.byref(prob), _tensor(q), _tensor(k_spec), _tensor(v_spec), Sk_spec,
                                    int(bool(causal_spec)), _tensor(k), _tensor(v), ctypes.byref(pat), _tensor(out),
                                    _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check("bsa_speculative_sparse", st)
    return out, lse


def speculative_sparse_noalloc(q, k_spec, v_spec, k, v, missed: BlockPattern, *, out: torch.Tensor,
                               lse: Optional[torch.Tensor] = None, causal_spec: bool = True, softmax_scale=None,
                               softcap: float = 0.0, stream=None):
    """``speculative_sparse`` without any device allocation: the caller passes the outputs
    (``out`` like q, bf16 or float32; ``lse`` float32 [B, Hq, Sq] or None) and the partials
    live in the library's per-device scratch area (NOALLOC_SCRATCH_BYTES).  Calls that
    overlap on one GPU share that area and race.  Returns (out, lse)."""
    lib = load()
    prob = _problem(q, k, False, softmax_scale, softcap=softcap)
    pat = missed.struct(prob.Hq)
    st = lib.bsa_speculative_sparse_noalloc(ctypes.byref(prob), _tensor(q), _tensor(k_spec), _tensor(v_spec),
                                            k_spec.shape[1], int(bool(causal_spec)), _tensor(k), _tensor(v),
                                            ctypes.byref(pat), _tensor(out), _ptr(lse), _stream(stream))
    _check("bsa_speculative_sparse_noalloc", st)
    return out, lse
