"""Thin Python binding of libdsa.so (the C ABI in include/dsa.h).

Argument marshalling only: every tensor, inputs and caller-supplied outputs and
workspaces alike, is checked for dtype, shape (outputs exactly, workspaces for
their byte size), device and contiguity before the library is called, and the
device pointers are handed to the library together with torch's current HIP
stream.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

IDX_HEADS, IDX_DIM = 32, 128
HEADS, D_NOPE, D_ROPE, D_V, D_LAT = 64, 192, 64, 256, 512
D_KV = D_LAT + D_ROPE
INDEX_TOPK = 2048  # index_topk of the configuration tables (default k)
MAX_TOPK = 8192    # largest k the library accepts
DEFAULT_SCALE = 1.0 / 16.0

OP_INDEX_SCORES, OP_TOPK, OP_SPARSE_MLA, OP_FORWARD = 0, 1, 2, 3
NO_WORKSPACE = "no-workspace"  # dsa_topk(ws=NO_WORKSPACE): pass NULL (one workgroup per row)
OUT_BF16, OUT_F32 = 0, 1
KV_BF16, KV_INT4 = 0, 1
KV_INT4_ROW_BYTES = 400


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str, hip_error: int):
        super().__init__(f"{fn}: status {status} ({msg}); last hip error {hip_error}")
        self.status = status
        self.hip_error = hip_error


class _CBatch(ctypes.Structure):
    _fields_ = [
        ("num_queries", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("q_seq", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("seq_row0", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("max_pages", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
    ]


_lib = None

_P = ctypes.c_void_p
_SIGS = {
    "dsa_index_scores": ([ctypes.POINTER(_CBatch), _P, _P, _P, _P, ctypes.c_int64, _P], ctypes.c_int),
    "dsa_topk": ([ctypes.POINTER(_CBatch), _P, ctypes.c_int64, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P],
                 ctypes.c_int),
    "dsa_sparse_mla_attn": ([ctypes.POINTER(_CBatch), _P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_float,
                             _P, ctypes.c_int32, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "dsa_forward": ([ctypes.POINTER(_CBatch), _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_float,
                     _P, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "dsa_forward_noalloc": ([ctypes.POINTER(_CBatch), _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                             ctypes.c_float, _P, ctypes.c_int32, _P, _P], ctypes.c_int),
    "dsa_index_share_schedule": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P], ctypes.c_int),
    "dsa_quantize_kv_int4": ([_P, ctypes.c_int64, _P, _P], ctypes.c_int),
    "dsa_check_device_args": ([ctypes.POINTER(_CBatch), _P, ctypes.c_int32, ctypes.c_int64, _P, _P], ctypes.c_int),
    "dsa_last_device_arg_flags": ([], ctypes.c_uint32),
    "dsa_workspace_bytes": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32], ctypes.c_size_t),
    "dsa_status_string": ([ctypes.c_int32], ctypes.c_char_p),
    "dsa_abi_version": ([], ctypes.c_int32),
    "dsa_last_hip_error": ([], ctypes.c_int32),
}
EXPORTED = tuple(_SIGS)


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} not built: run `python -m long_context_sparse_index_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


ERR_DEVICE_ARGS = 8
ARG_Q_SEQ, ARG_Q_POS, ARG_CACHE_ROW, ARG_IDX = 1, 2, 4, 8


def _check(fn: str, status: int) -> None:
    if status != 0:
        L = lib()
        err = DsaError(fn, status, L.dsa_status_string(status).decode(), L.dsa_last_hip_error())
        err.arg_flags = int(L.dsa_last_device_arg_flags()) if status == ERR_DEVICE_ARGS else 0
        raise err


def _ptr(x: Optional[torch.Tensor]) -> Optional[int]:
    return None if x is None else x.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _bf16(x: torch.Tensor, name: str, shape) -> torch.Tensor:
    """bf16 bits (bfloat16, int16 or uint16), contiguous, on the device; `shape`
    a full shape, or (None, n) for [rows, n] with any number of rows."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor, got {type(x).__name__}")
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: expected bf16 bits, got {x.dtype}")
    if shape is not None:
        ok = x.dim() == len(shape) and all(s is None or int(a) == s for a, s in zip(x.shape, shape))
        if not ok:
            raise ValueError(f"{name}: shape {tuple(x.shape)} does not match {tuple(shape)}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")
    return x


def _int32_out(x: torch.Tensor, name: str, shape) -> torch.Tensor:
    """A caller-supplied int32 output array of exactly `shape`, contiguous, on the device."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.int32:
        raise ValueError(f"{name}: expected an int32 tensor")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(x.shape)} != {tuple(shape)}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")
    return x


def _out_tensor(out: torch.Tensor, T: int, od: int) -> torch.Tensor:
    """A caller-supplied attention output: [T, 64, 256] of the requested element type."""
    want = torch.float32 if od == OUT_F32 else torch.bfloat16
    if not isinstance(out, torch.Tensor) or out.dtype != want:
        raise ValueError(f"out: expected a {want} tensor (out_dtype), got "
                         f"{getattr(out, 'dtype', type(out).__name__)}")
    if tuple(out.shape) != (T, HEADS, D_V):
        raise ValueError(f"out: shape {tuple(out.shape)} != {(T, HEADS, D_V)}")
    if not out.is_cuda or not out.is_contiguous():
        raise ValueError("out: must be a contiguous device tensor")
    return out


def _scores_tensor(scores: torch.Tensor, T: int, max_ctx: int) -> torch.Tensor:
    """A score matrix: row-major fp32 on the device with at least T rows of max_ctx."""
    if not isinstance(scores, torch.Tensor) or scores.dtype != torch.float32 or scores.dim() != 2 \
            or scores.stride(1) != 1:
        raise ValueError("scores: expected a row-major 2-D fp32 tensor")
    if scores.shape[0] < T or scores.shape[1] < max_ctx:
        raise ValueError(f"scores: shape {tuple(scores.shape)} is smaller than ({T}, {max_ctx})")
    if not scores.is_cuda:
        raise ValueError("scores: must be a device tensor")
    return scores


def _workspace(ws: torch.Tensor, need: int) -> torch.Tensor:
    """A caller-supplied workspace: a contiguous device tensor of at least `need` bytes
    (any element type; its size is passed in bytes)."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws: must be a contiguous device tensor")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"ws: {ws.numel() * ws.element_size()} bytes < the {need} bytes needed")
    return ws


def _nbytes(ws: Optional[torch.Tensor]) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


class Batch:
    """Batch geometry: q_seq [T] int32 and q_pos [T] int32 on the device, and the
    cache layout: contiguous (seq_row0 [B] int64: first cache row of each
    sequence) or paged (block_table [B, max_pages] int32 page ids and
    page_size tokens per page; seq_row0 then None), and the latent cache's row
    format (KV_BF16: [rows, 576] bf16; KV_INT4: [rows, 400] uint8)."""

    def __init__(self, q_seq: torch.Tensor, q_pos: torch.Tensor, seq_row0: Optional[torch.Tensor], max_ctx: int,
                 block_table: Optional[torch.Tensor] = None, page_size: int = 0, kv_format: int = KV_BF16):
        for name, x, dt in (("q_seq", q_seq, torch.int32), ("q_pos", q_pos, torch.int32)):
            if x.dtype != dt or not x.is_cuda or not x.is_contiguous() or x.dim() != 1:
                raise ValueError(f"{name}: expected a contiguous 1-D {dt} device tensor")
        if q_seq.shape != q_pos.shape:
            raise ValueError("q_seq and q_pos differ in length")
        if page_size:
            if block_table is None or block_table.dtype != torch.int32 or not block_table.is_cuda \
                    or not block_table.is_contiguous() or block_table.dim() != 2:
                raise ValueError("block_table: expected a contiguous [B, max_pages] int32 device tensor")
            self.B = int(block_table.shape[0])
        else:
            if seq_row0 is None or seq_row0.dtype != torch.int64 or not seq_row0.is_cuda \
                    or not seq_row0.is_contiguous() or seq_row0.dim() != 1:
                raise ValueError("seq_row0: expected a contiguous 1-D int64 device tensor")
            self.B = int(seq_row0.shape[0])
        self.q_seq, self.q_pos, self.seq_row0 = q_seq, q_pos, seq_row0
        self.block_table, self.page_size = block_table, int(page_size)
        self.kv_format = int(kv_format)
        self.max_ctx = int(max_ctx)
        self.T = int(q_seq.shape[0])

    def c(self) -> _CBatch:
        mp = int(self.block_table.shape[1]) if self.page_size else 0
        return _CBatch(self.T, self.B, self.max_ctx, self.page_size, _ptr(self.q_seq), _ptr(self.q_pos),
                       _ptr(self.seq_row0), _ptr(self.block_table), mp, self.kv_format)

    def slice(self, t0: int, t1: int) -> "Batch":
        return Batch(self.q_seq[t0:t1], self.q_pos[t0:t1], self.seq_row0, self.max_ctx, self.block_table,
                     self.page_size, self.kv_format)


def _kv(batch: "Batch", kv: torch.Tensor) -> torch.Tensor:
    if batch.kv_format == KV_INT4:
        if kv.dtype != torch.uint8 or not kv.is_cuda or not kv.is_contiguous() or kv.dim() != 2 \
                or kv.shape[1] != KV_INT4_ROW_BYTES:
            raise ValueError(f"kv: expected a contiguous [rows, {KV_INT4_ROW_BYTES}] uint8 device tensor (INT4 rows)")
        return kv
    return _bf16(kv, "kv", (None, D_KV))


def dsa_quantize_kv_int4(kv: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 latent-cache rows [rows, 576] -> INT4 rows [rows, 400] uint8."""
    _bf16(kv, "kv", (None, D_KV))
    if out is None:
        out = torch.empty((kv.shape[0], KV_INT4_ROW_BYTES), dtype=torch.uint8, device=kv.device)
    elif out.dtype != torch.uint8 or tuple(out.shape) != (kv.shape[0], KV_INT4_ROW_BYTES) \
            or not out.is_cuda or not out.is_contiguous():
        raise ValueError(f"out: expected a contiguous [{kv.shape[0]}, {KV_INT4_ROW_BYTES}] uint8 device tensor")
    _check("dsa_quantize_kv_int4", lib().dsa_quantize_kv_int4(_ptr(kv), kv.shape[0], _ptr(out), _stream()))
    return out


def _out_dtype(out_dtype) -> int:
    if out_dtype == torch.float32:
        return OUT_F32
    if out_dtype == torch.bfloat16:
        return OUT_BF16
    raise ValueError(f"out_dtype: expected torch.bfloat16 or torch.float32, got {out_dtype}")


def score_ld(max_ctx: int) -> int:
    return (max_ctx + 3) // 4 * 4


def dsa_workspace_bytes(op: int, num_queries: int, max_ctx: int, k: int) -> int:
    return int(lib().dsa_workspace_bytes(op, num_queries, max_ctx, k))


def dsa_index_share_schedule(num_layers: int = 78, num_dense: int = 3, index_topk_freq: int = 4) -> list:
    """IndexShare schedule: source[l] == l for a layer that runs its own indexer
    and top-k, else the earlier full layer whose selection layer l reuses."""
    src = (ctypes.c_int32 * max(num_layers, 1))()
    _check("dsa_index_share_schedule",
           lib().dsa_index_share_schedule(num_layers, num_dense, index_topk_freq, src))
    return list(src[:num_layers])


def dsa_index_scores(batch: Batch, q_idx, w, k_idx, scores: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexer scores [T, ld] fp32 (only s <= q_pos[t] written)."""
    T = batch.T
    _bf16(q_idx, "q_idx", (T, IDX_HEADS, IDX_DIM))
    _bf16(w, "w", (T, IDX_HEADS))
    _bf16(k_idx, "k_idx", (None, IDX_DIM))
    if scores is None:
        scores = torch.empty((T, score_ld(batch.max_ctx)), dtype=torch.float32, device=q_idx.device)
    _scores_tensor(scores, T, batch.max_ctx)
    cb = batch.c()
    _check("dsa_index_scores", lib().dsa_index_scores(ctypes.byref(cb), _ptr(q_idx), _ptr(w), _ptr(k_idx),
                                                      _ptr(scores), scores.stride(0), _stream()))
    return scores


def dsa_topk(batch: Batch, scores: torch.Tensor, k: int = INDEX_TOPK,
             idx: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k positions [T, k] int32, ascending, -1 padded."""
    _scores_tensor(scores, batch.T, batch.max_ctx)
    if not 1 <= k <= MAX_TOPK:
        raise ValueError(f"k: {k} outside 1..{MAX_TOPK}")
    if idx is None:
        idx = torch.empty((batch.T, k), dtype=torch.int32, device=scores.device)
    _int32_out(idx, "idx", (batch.T, k))
    need = dsa_workspace_bytes(OP_TOPK, batch.T, batch.max_ctx, k)
    if isinstance(ws, str) and ws == NO_WORKSPACE:
        ws = None
    elif ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device) if need else None
    else:
        _workspace(ws, need)
    cb = batch.c()
    _check("dsa_topk", lib().dsa_topk(ctypes.byref(cb), _ptr(scores), scores.stride(0), k, _ptr(idx),
                                      _ptr(ws), _nbytes(ws), _stream()))
    return idx


def dsa_sparse_mla_attn(batch: Batch, q_nope, q_rope, kv, w_uk, w_uv, idx: torch.Tensor,
                        softmax_scale: float = DEFAULT_SCALE, out_dtype=torch.bfloat16,
                        out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sparse MLA output [T, 64, 256] over the positions in idx (-1 = absent)."""
    T = batch.T
    _bf16(q_nope, "q_nope", (T, HEADS, D_NOPE))
    _bf16(q_rope, "q_rope", (T, HEADS, D_ROPE))
    _kv(batch, kv)
    _bf16(w_uk, "w_uk", (HEADS, D_LAT, D_NOPE))
    _bf16(w_uv, "w_uv", (HEADS, D_LAT, D_V))
    if not isinstance(idx, torch.Tensor) or idx.dim() != 2 or not 1 <= int(idx.shape[1]) <= MAX_TOPK:
        raise ValueError(f"idx: expected a [T, k] int32 tensor with 1 <= k <= {MAX_TOPK}")
    k = int(idx.shape[1])
    _int32_out(idx, "idx", (T, k))
    od = _out_dtype(out_dtype)
    if out is None:
        out = torch.empty((T, HEADS, D_V), dtype=torch.float32 if od else torch.bfloat16, device=kv.device)
    _out_tensor(out, T, od)
    need = dsa_workspace_bytes(OP_SPARSE_MLA, T, batch.max_ctx, k)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=kv.device)
    else:
        _workspace(ws, need)
    cb = batch.c()
    _check("dsa_sparse_mla_attn",
           lib().dsa_sparse_mla_attn(ctypes.byref(cb), _ptr(q_nope), _ptr(q_rope), _ptr(kv), _ptr(w_uk), _ptr(w_uv),
                                     _ptr(idx), k, softmax_scale, _ptr(out), od, _ptr(ws), _nbytes(ws), _stream()))
    return out


def dsa_forward(batch: Batch, q_idx, w, k_idx, q_nope, q_rope, kv, w_uk, w_uv, k: int = INDEX_TOPK,
                softmax_scale: float = DEFAULT_SCALE, out_dtype=torch.bfloat16, return_idx: bool = True,
                ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                idx: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Indexer -> top-k -> sparse MLA.  Returns (out [T,64,256], idx [T,k] or None)."""
    T = batch.T
    _bf16(q_idx, "q_idx", (T, IDX_HEADS, IDX_DIM))
    _bf16(w, "w", (T, IDX_HEADS))
    _bf16(k_idx, "k_idx", (None, IDX_DIM))
    _bf16(q_nope, "q_nope", (T, HEADS, D_NOPE))
    _bf16(q_rope, "q_rope", (T, HEADS, D_ROPE))
    _kv(batch, kv)
    _bf16(w_uk, "w_uk", (HEADS, D_LAT, D_NOPE))
    _bf16(w_uv, "w_uv", (HEADS, D_LAT, D_V))
    if not 1 <= k <= MAX_TOPK:
        raise ValueError(f"k: {k} outside 1..{MAX_TOPK}")
    od = _out_dtype(out_dtype)
    if out is None:
        out = torch.empty((T, HEADS, D_V), dtype=torch.float32 if od else torch.bfloat16, device=kv.device)
    _out_tensor(out, T, od)
    if return_idx:
        if idx is None:
            idx = torch.empty((T, k), dtype=torch.int32, device=kv.device)
        _int32_out(idx, "idx", (T, k))
    if ws is None:
        need = dsa_workspace_bytes(OP_FORWARD, T, batch.max_ctx, k)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=kv.device)
    else:  # a smaller workspace runs the queries in chunks; one query must fit
        _workspace(ws, dsa_workspace_bytes(OP_FORWARD, min(T, 1), batch.max_ctx, k))
    cb = batch.c()
    _check("dsa_forward",
           lib().dsa_forward(ctypes.byref(cb), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(q_nope), _ptr(q_rope),
                             _ptr(kv), _ptr(w_uk), _ptr(w_uv), k, softmax_scale, _ptr(out), od,
                             _ptr(idx) if return_idx else None, _ptr(ws), _nbytes(ws), _stream()))
    return out, (idx if return_idx else None)


def dsa_forward_noalloc(batch: Batch, q_idx, w, k_idx, q_nope, q_rope, kv, w_uk, w_uv, out: torch.Tensor,
                        idx: Optional[torch.Tensor] = None, k: int = INDEX_TOPK,
                        softmax_scale: float = DEFAULT_SCALE) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """dsa_forward over the library's static per-device scratch (no workspace; the
    library allocates nothing).  The caller supplies `out` [T, 64, 256] (bf16 or
    fp32, which selects the output type) and optionally `idx` [T, k] int32; this
    wrapper allocates nothing either.  Calls overlapping on one device race."""
    T = batch.T
    _bf16(q_idx, "q_idx", (T, IDX_HEADS, IDX_DIM))
    _bf16(w, "w", (T, IDX_HEADS))
    _bf16(k_idx, "k_idx", (None, IDX_DIM))
    _bf16(q_nope, "q_nope", (T, HEADS, D_NOPE))
    _bf16(q_rope, "q_rope", (T, HEADS, D_ROPE))
    _kv(batch, kv)
    _bf16(w_uk, "w_uk", (HEADS, D_LAT, D_NOPE))
    _bf16(w_uv, "w_uv", (HEADS, D_LAT, D_V))
    if not 1 <= k <= MAX_TOPK:
        raise ValueError(f"k: {k} outside 1..{MAX_TOPK}")
    if not isinstance(out, torch.Tensor):
        raise ValueError("out: the caller supplies the output tensor")
    od = _out_dtype(out.dtype)
    _out_tensor(out, T, od)
    if idx is not None:
        _int32_out(idx, "idx", (T, k))
    cb = batch.c()
    _check("dsa_forward_noalloc",
           lib().dsa_forward_noalloc(ctypes.byref(cb), _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(q_nope),
                                     _ptr(q_rope), _ptr(kv), _ptr(w_uk), _ptr(w_uv), k, softmax_scale,
                                     _ptr(out), od, _ptr(idx), _stream()))
    return out, idx


def dsa_check_device_args(batch: Batch, idx: Optional[torch.Tensor] = None, cache_rows: int = 0,
                          flags: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device-side argument check: a 1-element int32 device tensor holding the
    ARG_* bits of every violated device-side precondition (0 when all hold)."""
    if idx is not None:
        if not isinstance(idx, torch.Tensor) or idx.dtype != torch.int32 or idx.dim() != 2 \
                or idx.shape[0] != batch.T or not idx.is_cuda or not idx.is_contiguous():
            raise ValueError("idx: expected a contiguous [T, k] int32 device tensor")
    if flags is None:
        flags = torch.empty(1, dtype=torch.int32, device=batch.q_seq.device)
    _int32_out(flags, "flags", (1,))
    cb = batch.c()
    _check("dsa_check_device_args",
           lib().dsa_check_device_args(ctypes.byref(cb), _ptr(idx), 0 if idx is None else int(idx.shape[1]),
                                       int(cache_rows), _ptr(flags), _stream()))
    return flags
