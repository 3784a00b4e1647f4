"""Python binding of libmsa (include/msa.h): MiniMax Sparse Attention on MI355X.

Argument marshalling only. Every step of the path runs in the HIP kernels of
libmsa.so; torch supplies device memory and the current stream. There is no
fallback: if the library is missing or a call fails, an exception is raised.

Entry points (same names as the C ABI): every function of include/msa.h (the
EXPORTS table), plus helpers that allocate outputs and run the whole path:
  prefill(...), decode(...), decode_per_token(...) and prefill_tokens(...).
"""

import ctypes
import dataclasses
import pathlib
from typing import Optional

import numpy as np
import torch

_LIB_PATH = pathlib.Path(__file__).resolve().parent / "libmsa.so"
_lib = None

MSA_F32, MSA_BF16 = 0, 1
MSA_CACHE_PLAIN, MSA_CACHE_FP8_E4M3 = 0, 1
BLOCK = 128
SCALE_BLOCK = 32      # channels per FP8 scale


class MsaError(RuntimeError):
    """A libmsa call returned a non-zero status."""

    def __init__(self, status, message):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_q_heads", "num_kv_heads", "head_dim", "num_idx_heads", "idx_head_dim",
        "num_sel_groups", "block_size", "dtype", "cache_format")]


class _Cache(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("k_idx_cache", ctypes.c_void_p), ("num_phys_blocks", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("num_seqs", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_idx_scale", ctypes.c_void_p)]


class _Unit(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("r", "tau", "row0", "num_rows", "pos0")]


class _Batch(ctypes.Structure):
    _fields_ = [("units", ctypes.c_void_p), ("total_units", ctypes.c_int32),
                ("total_q", ctypes.c_int32)]


EXPORTS = {
    # name: (restype, argtypes)
    "msa_prefill_plan": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "msa_index_scores": (ctypes.c_int, [ctypes.POINTER(_Geom), ctypes.POINTER(_Cache),
                                        ctypes.POINTER(_Batch), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "msa_select_topk_blocks": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "msa_sparse_attn_prefill": (ctypes.c_int, [ctypes.POINTER(_Geom), ctypes.POINTER(_Cache),
                                               ctypes.POINTER(_Batch), ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                                               ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p]),
    "msa_prefill_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(_Geom),
                                                     ctypes.POINTER(_Cache), ctypes.c_int32,
                                                     ctypes.c_int32]),
    "msa_sparse_attn_prefill_staged": (ctypes.c_int, [
        ctypes.POINTER(_Geom), ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "msa_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(_Geom), ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_int32]),
    "msa_sparse_attn_decode": (ctypes.c_int, [ctypes.POINTER(_Geom), ctypes.POINTER(_Cache),
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_float, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "msa_sparse_attn_decode_static": (ctypes.c_int, [
        ctypes.POINTER(_Geom), ctypes.POINTER(_Cache), ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]),
    "msa_qk_norm_rope_insert": (ctypes.c_int, [ctypes.POINTER(_Geom), ctypes.POINTER(_Cache),
                                               ctypes.POINTER(_Batch), ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
                                               ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_void_p]),
    "msa_index_scores_per_token": (ctypes.c_int, [ctypes.POINTER(_Geom), ctypes.POINTER(_Cache),
                                                  ctypes.c_int32, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p]),
    "msa_sparse_attn_decode_per_token": (ctypes.c_int, [
        ctypes.POINTER(_Geom), ctypes.POINTER(_Cache), ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "msa_index_scores_prefill_tokens": (ctypes.c_int, [
        ctypes.POINTER(_Geom), ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p]),
    "msa_prefill_tokens_workspace_size": (ctypes.c_size_t, [
        ctypes.POINTER(_Geom), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "msa_sparse_attn_prefill_tokens": (ctypes.c_int, [
        ctypes.POINTER(_Geom), ctypes.POINTER(_Cache), ctypes.POINTER(_Batch), ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "msa_validate_block_table": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]),
    "msa_validate_ids": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32]),
    "msa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "msa_last_error": (ctypes.c_char_p, []),
    "msa_version": (ctypes.c_int32, []),
}


def lib():
    """The loaded libmsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m block_sparse_long_11_amd.build` (there is no fallback path)")
        handle = ctypes.CDLL(str(_LIB_PATH))
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def lib_path():
    return _LIB_PATH


def _status_name(status):
    try:
        return lib().msa_status_string(status).decode()
    except Exception:   # library unavailable while formatting an error
        return f"status {status}"


def _check(status):
    if status != 0:
        raise MsaError(status, lib().msa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


@dataclasses.dataclass
class Geometry:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_idx_heads: int
    idx_head_dim: int
    num_sel_groups: int
    dtype: str = "bf16"          # "bf16" or "f32"
    cache_format: str = "plain"  # "plain" (caches in dtype) or "fp8" (E4M3 + scales)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def fp8(self):
        return self.cache_format == "fp8"

    @property
    def cache_torch_dtype(self):
        return torch.uint8 if self.fp8 else self.torch_dtype

    def c(self):
        return _Geom(self.num_q_heads, self.num_kv_heads, self.head_dim, self.num_idx_heads,
                     self.idx_head_dim, self.num_sel_groups, BLOCK,
                     MSA_BF16 if self.dtype == "bf16" else MSA_F32,
                     MSA_CACHE_FP8_E4M3 if self.fp8 else MSA_CACHE_PLAIN)


@dataclasses.dataclass
class Cache:
    """Block-major paged caches on one device (see include/msa.h). With FP8 caches
    the three caches are uint8 E4M3 codes and the scale tensors are set."""
    k_cache: torch.Tensor        # [P][H_kv][128][D]
    v_cache: torch.Tensor        # [P][H_kv][D][128] (each block d-major)
    k_idx_cache: torch.Tensor    # [P][H_i][128][D_i]
    block_table: torch.Tensor    # int32 [B][max_blocks]
    seq_lens: torch.Tensor       # int32 [B]
    k_scale: Optional[torch.Tensor] = None       # uint8 [P][H_kv][128][D/32]
    v_scale: Optional[torch.Tensor] = None       # uint8 [P][H_kv][D/32][128]
    k_idx_scale: Optional[torch.Tensor] = None   # uint8 [P][H_i][128][D_i/32]

    def check(self, geom: Geometry):
        dt, dev = geom.cache_torch_dtype, self.block_table.device
        _need(self.k_cache, "k_cache", dt, 4, dev)
        _need(self.v_cache, "v_cache", dt, 4, dev)
        _need(self.k_idx_cache, "k_idx_cache", dt, 4, dev)
        _need(self.block_table, "block_table", torch.int32, 2, dev)
        _need(self.seq_lens, "seq_lens", torch.int32, 1, dev)
        P = self.k_cache.shape[0]
        if tuple(self.k_cache.shape) != (P, geom.num_kv_heads, BLOCK, geom.head_dim):
            raise ValueError("k_cache must be [P][H_kv][128][D]")
        if tuple(self.v_cache.shape) != (P, geom.num_kv_heads, geom.head_dim, BLOCK):
            raise ValueError("v_cache must be [P][H_kv][D][128] (d-major blocks)")
        if tuple(self.k_idx_cache.shape) != (P, geom.num_idx_heads, BLOCK, geom.idx_head_dim):
            raise ValueError("k_idx_cache must be [P][H_i][128][D_i]")
        if self.seq_lens.shape[0] != self.block_table.shape[0]:
            raise ValueError("seq_lens and block_table disagree on the number of sequences")
        if geom.fp8:
            H, D, Hi, Di = geom.num_kv_heads, geom.head_dim, geom.num_idx_heads, geom.idx_head_dim
            for t, name, shape in ((self.k_scale, "k_scale", (P, H, BLOCK, D // SCALE_BLOCK)),
                                   (self.v_scale, "v_scale", (P, H, D // SCALE_BLOCK, BLOCK)),
                                   (self.k_idx_scale, "k_idx_scale",
                                    (P, Hi, BLOCK, Di // SCALE_BLOCK))):
                _need(t, name, torch.uint8, 4, dev)
                if tuple(t.shape) != shape:
                    raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")

    @property
    def num_seqs(self):
        return self.block_table.shape[0]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]

    def c(self):
        sp = lambda t: None if t is None else t.data_ptr()
        return _Cache(self.k_cache.data_ptr(), self.v_cache.data_ptr(),
                      self.k_idx_cache.data_ptr(), self.k_cache.shape[0],
                      self.block_table.data_ptr(), self.block_table.shape[1],
                      self.seq_lens.data_ptr(), self.block_table.shape[0],
                      sp(self.k_scale), sp(self.v_scale), sp(self.k_idx_scale))


@dataclasses.dataclass
class Batch:
    """A planned prefill batch: `units` (host int32 [U][5]) and its device copy."""
    units_host: np.ndarray
    units: torch.Tensor          # int32 [U][5] on the device
    total_q: int

    @property
    def total_units(self):
        return int(self.units_host.shape[0])

    def c(self):
        return _Batch(self.units.data_ptr() if self.total_units else None,
                      self.total_units, self.total_q)


# ----------------------------------------------------------------------------
# C-ABI wrappers
# ----------------------------------------------------------------------------

def msa_prefill_plan(seq_lens, q_lens):
    """Host plan of a prefill batch: int32 [U][5] rows (r, tau, row0, num_rows, pos0)."""
    sl = _host_int32(seq_lens, "seq_lens", 1)
    ql = _host_int32(q_lens, "q_lens", 1)
    if sl.shape != ql.shape:
        raise ValueError("seq_lens and q_lens must be of equal length")
    n = ctypes.c_int32(0)
    _check(lib().msa_prefill_plan(sl.ctypes.data, ql.ctypes.data, len(sl), None, 0,
                                  ctypes.byref(n)))
    units = np.zeros((n.value, 5), dtype=np.int32)
    _check(lib().msa_prefill_plan(sl.ctypes.data, ql.ctypes.data, len(sl),
                                  units.ctypes.data if n.value else None, n.value,
                                  ctypes.byref(n)))
    return units


def make_batch(seq_lens, q_lens, device):
    units = msa_prefill_plan(seq_lens, q_lens)
    return Batch(units, torch.from_numpy(units).to(device), int(np.sum(q_lens)))


def msa_index_scores(geom: Geometry, cache: Cache, batch, q_idx, scores, stream=None):
    """Step 1. batch=None is decode. scores: fp32 [U][n_sel][max_blocks]."""
    cache.check(geom)
    dev = cache.block_table.device
    _need(q_idx, "q_idx", geom.torch_dtype, 3, dev)
    _need(scores, "scores", torch.float32, 3, dev)
    U = cache.num_seqs if batch is None else batch.total_units
    rows_q = cache.num_seqs if batch is None else batch.total_q
    if tuple(q_idx.shape) != (rows_q, geom.num_idx_heads, geom.idx_head_dim):
        raise ValueError(f"q_idx must be [{rows_q}][H_i][D_i], got {tuple(q_idx.shape)}")
    if tuple(scores.shape) != (U, geom.num_sel_groups, cache.max_blocks):
        raise ValueError(f"scores must be [{U}][n_sel][{cache.max_blocks}]")
    g, c = geom.c(), cache.c()
    b = None if batch is None else ctypes.pointer(batch.c())
    _check(lib().msa_index_scores(ctypes.byref(g), ctypes.byref(c), b, _ptr(q_idx),
                                  _ptr(scores), _stream(stream)))


def msa_select_topk_blocks(scores, topk, ids, stream=None):
    """Step 2 over the rows of scores (any leading shape); ids int32 [..., topk]."""
    _need(scores, "scores", torch.float32)
    _need(ids, "ids", torch.int32, None, scores.device)
    row_len = scores.shape[-1]
    rows = scores.numel() // row_len
    if ids.numel() != rows * topk or ids.shape[-1] != topk:
        raise ValueError("ids must hold [rows][topk]")
    _check(lib().msa_select_topk_blocks(_ptr(scores), rows, row_len, topk, _ptr(ids),
                                        _stream(stream)))


def _check_prefill_attn(geom, cache, batch, q, ids, topk, out, lse):
    cache.check(geom)
    dev = cache.block_table.device
    _need(q, "q", geom.torch_dtype, 3, dev)
    _need(out, "out", geom.torch_dtype, 3, dev)
    _need(ids, "ids", torch.int32, 3, dev)
    shape = (batch.total_q, geom.num_q_heads, geom.head_dim)
    if tuple(q.shape) != shape or tuple(out.shape) != shape:
        raise ValueError(f"q and out must be {shape}")
    if tuple(ids.shape) != (batch.total_units, geom.num_sel_groups, topk):
        raise ValueError("ids must be [U][n_sel][topk]")
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != shape[:2]:
            raise ValueError("lse must be [total_q][H_q]")


def msa_sparse_attn_prefill(geom: Geometry, cache: Cache, batch: Batch, q, ids, topk, out,
                            lse=None, softmax_scale=0.0, stream=None):
    """Step 3 for prefill. q/out [total_q][H_q][D], lse fp32 [total_q][H_q] or None."""
    _check_prefill_attn(geom, cache, batch, q, ids, topk, out, lse)
    g, c, b = geom.c(), cache.c(), batch.c()
    _check(lib().msa_sparse_attn_prefill(ctypes.byref(g), ctypes.byref(c), ctypes.byref(b),
                                         _ptr(q), _ptr(ids), topk, float(softmax_scale),
                                         _ptr(out), _ptr(lse), _stream(stream)))


def msa_prefill_workspace_size(geom: Geometry, cache: Cache, total_units, topk):
    g, c = geom.c(), cache.c()
    return int(lib().msa_prefill_workspace_size(ctypes.byref(g), ctypes.byref(c), total_units,
                                                topk))


def msa_sparse_attn_prefill_staged(geom: Geometry, cache: Cache, batch: Batch, q, ids, topk,
                                   out, workspace, lse=None, softmax_scale=0.0, stream=None):
    """Step 3 for prefill with a workspace (FP8 caches: kept blocks converted to bf16
    once each, then the bf16 attention)."""
    _check_prefill_attn(geom, cache, batch, q, ids, topk, out, lse)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, cache.block_table.device)
    g, c, b = geom.c(), cache.c(), batch.c()
    _check(lib().msa_sparse_attn_prefill_staged(
        ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), _ptr(q), _ptr(ids), topk,
        float(softmax_scale), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _ptr(out), _ptr(lse), _stream(stream)))


def msa_decode_workspace_size(geom: Geometry, num_seqs, topk, num_splits=0):
    g = geom.c()
    return int(lib().msa_decode_workspace_size(ctypes.byref(g), num_seqs, topk, num_splits))


def msa_sparse_attn_decode(geom: Geometry, cache: Cache, q, ids, topk, out, workspace,
                           lse=None, num_splits=0, softmax_scale=0.0, stream=None):
    """Steps 3+4 for decode. q/out [B][H_q][D]; workspace a uint8 device tensor."""
    cache.check(geom)
    dev = cache.block_table.device
    B = cache.num_seqs
    _need(q, "q", geom.torch_dtype, 3, dev)
    _need(out, "out", geom.torch_dtype, 3, dev)
    _need(ids, "ids", torch.int32, 3, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    shape = (B, geom.num_q_heads, geom.head_dim)
    if tuple(q.shape) != shape or tuple(out.shape) != shape:
        raise ValueError(f"q and out must be {shape}")
    if tuple(ids.shape) != (B, geom.num_sel_groups, topk):
        raise ValueError("ids must be [B][n_sel][topk]")
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    g, c = geom.c(), cache.c()
    _check(lib().msa_sparse_attn_decode(ctypes.byref(g), ctypes.byref(c), _ptr(q), _ptr(ids),
                                        topk, float(softmax_scale), num_splits, _ptr(workspace),
                                        workspace.numel(), _ptr(out), _ptr(lse),
                                        _stream(stream)))


STATIC_SCRATCH_BYTES = 16 * 1024 * 1024   # MSA_STATIC_SCRATCH_BYTES


def msa_sparse_attn_decode_static(geom: Geometry, cache: Cache, q, ids, topk, out, lse=None,
                                  num_splits=0, softmax_scale=0.0, stream=None):
    """msa_sparse_attn_decode without a workspace: the library's static scratch
    holds the split partials (for callers that cannot allocate)."""
    cache.check(geom)
    dev = cache.block_table.device
    B = cache.num_seqs
    _need(q, "q", geom.torch_dtype, 3, dev)
    _need(out, "out", geom.torch_dtype, 3, dev)
    _need(ids, "ids", torch.int32, 3, dev)
    shape = (B, geom.num_q_heads, geom.head_dim)
    if tuple(q.shape) != shape or tuple(out.shape) != shape:
        raise ValueError(f"q and out must be {shape}")
    if tuple(ids.shape) != (B, geom.num_sel_groups, topk):
        raise ValueError("ids must be [B][n_sel][topk]")
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    g, c = geom.c(), cache.c()
    _check(lib().msa_sparse_attn_decode_static(ctypes.byref(g), ctypes.byref(c), _ptr(q),
                                               _ptr(ids), topk, float(softmax_scale),
                                               num_splits, _ptr(out), _ptr(lse),
                                               _stream(stream)))


def msa_qk_norm_rope_insert(geom: Geometry, cache: Cache, batch, q, k, v, k_idx, q_norm_w,
                            k_norm_w, eps, rope_theta, rotary_dim, q_out=None, stream=None):
    """Step 0: QK-norm + partial RoPE of the new tokens; K, V and k_idx go into the
    caches. batch=None is decode (row r = sequence r at position seq_lens[r]-1).
    q/q_out [rows][H_q][D] (q_out=None: in place), k/v [rows][H_kv][D],
    k_idx [rows][H_i][D_i], q_norm_w/k_norm_w [D]."""
    cache.check(geom)
    dev, dt = cache.block_table.device, geom.torch_dtype
    rows = cache.num_seqs if batch is None else batch.total_q
    if q_out is None:
        q_out = q
    for t, name, shape in ((q, "q", (rows, geom.num_q_heads, geom.head_dim)),
                           (q_out, "q_out", (rows, geom.num_q_heads, geom.head_dim)),
                           (k, "k", (rows, geom.num_kv_heads, geom.head_dim)),
                           (v, "v", (rows, geom.num_kv_heads, geom.head_dim)),
                           (k_idx, "k_idx", (rows, geom.num_idx_heads, geom.idx_head_dim)),
                           (q_norm_w, "q_norm_w", (geom.head_dim,)),
                           (k_norm_w, "k_norm_w", (geom.head_dim,))):
        _need(t, name, dt, len(shape), dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    g, c = geom.c(), cache.c()
    b = None if batch is None else ctypes.pointer(batch.c())
    _check(lib().msa_qk_norm_rope_insert(ctypes.byref(g), ctypes.byref(c), b, _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(k_idx), _ptr(q_norm_w), _ptr(k_norm_w),
                                         float(eps), float(rope_theta), int(rotary_dim),
                                         _ptr(q_out), _stream(stream)))
    return q_out


def msa_index_scores_per_token(geom: Geometry, cache: Cache, tokens_per_seq, q_idx, scores,
                               stream=None):
    """Per-token decode indexer: q_idx [B*T][H_i][D_i] -> scores [B*T][n_sel][max_blocks]."""
    cache.check(geom)
    dev = cache.block_table.device
    rows = cache.num_seqs * tokens_per_seq
    _need(q_idx, "q_idx", geom.torch_dtype, 3, dev)
    _need(scores, "scores", torch.float32, 3, dev)
    if tuple(q_idx.shape) != (rows, geom.num_idx_heads, geom.idx_head_dim):
        raise ValueError(f"q_idx must be [{rows}][H_i][D_i]")
    if tuple(scores.shape) != (rows, geom.num_sel_groups, cache.max_blocks):
        raise ValueError(f"scores must be [{rows}][n_sel][{cache.max_blocks}]")
    g, c = geom.c(), cache.c()
    _check(lib().msa_index_scores_per_token(ctypes.byref(g), ctypes.byref(c), tokens_per_seq,
                                            _ptr(q_idx), _ptr(scores), _stream(stream)))


def msa_sparse_attn_decode_per_token(geom: Geometry, cache: Cache, tokens_per_seq, q, ids, topk,
                                     out, workspace, lse=None, num_splits=0, softmax_scale=0.0,
                                     stream=None):
    """Per-token decode attention: q/out [B*T][H_q][D], ids [B*T][n_sel][topk]."""
    cache.check(geom)
    dev = cache.block_table.device
    rows = cache.num_seqs * tokens_per_seq
    _need(q, "q", geom.torch_dtype, 3, dev)
    _need(out, "out", geom.torch_dtype, 3, dev)
    _need(ids, "ids", torch.int32, 3, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    shape = (rows, geom.num_q_heads, geom.head_dim)
    if tuple(q.shape) != shape or tuple(out.shape) != shape:
        raise ValueError(f"q and out must be {shape}")
    if tuple(ids.shape) != (rows, geom.num_sel_groups, topk):
        raise ValueError("ids must be [B*T][n_sel][topk]")
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    g, c = geom.c(), cache.c()
    _check(lib().msa_sparse_attn_decode_per_token(
        ctypes.byref(g), ctypes.byref(c), tokens_per_seq, _ptr(q), _ptr(ids), topk,
        float(softmax_scale), num_splits, _ptr(workspace), workspace.numel(), _ptr(out),
        _ptr(lse), _stream(stream)))


def decode_per_token(geom: Geometry, cache: Cache, tokens_per_seq, q, q_idx, topk, num_splits=0,
                     softmax_scale=0.0, stream=None):
    """Index, select and attend T new tokens per sequence, each with its own blocks."""
    dev = q.device
    rows = cache.num_seqs * tokens_per_seq
    scores = torch.empty((rows, geom.num_sel_groups, cache.max_blocks), dtype=torch.float32,
                         device=dev)
    ids = torch.empty((rows, geom.num_sel_groups, topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws = workspace(msa_decode_workspace_size(geom, rows, topk, num_splits), dev)
    msa_index_scores_per_token(geom, cache, tokens_per_seq, q_idx, scores, stream)
    msa_select_topk_blocks(scores, topk, ids, stream)
    msa_sparse_attn_decode_per_token(geom, cache, tokens_per_seq, q, ids, topk, out, ws, lse,
                                     num_splits, softmax_scale, stream)
    return dict(scores=scores, ids=ids, out=out, lse=lse)


def msa_index_scores_prefill_tokens(geom: Geometry, cache: Cache, batch: Batch, q_idx, scores,
                                    stream=None):
    """Per-token prefill indexer: q_idx [total_q][H_i][D_i] -> scores
    [total_q][n_sel][max_blocks], one row per new token."""
    cache.check(geom)
    dev = cache.block_table.device
    _need(q_idx, "q_idx", geom.torch_dtype, 3, dev)
    _need(scores, "scores", torch.float32, 3, dev)
    if tuple(q_idx.shape) != (batch.total_q, geom.num_idx_heads, geom.idx_head_dim):
        raise ValueError(f"q_idx must be [{batch.total_q}][H_i][D_i]")
    if tuple(scores.shape) != (batch.total_q, geom.num_sel_groups, cache.max_blocks):
        raise ValueError(f"scores must be [{batch.total_q}][n_sel][{cache.max_blocks}]")
    g, c, b = geom.c(), cache.c(), batch.c()
    _check(lib().msa_index_scores_prefill_tokens(ctypes.byref(g), ctypes.byref(c),
                                                 ctypes.byref(b), _ptr(q_idx), _ptr(scores),
                                                 _stream(stream)))


def msa_prefill_tokens_workspace_size(geom: Geometry, total_units, total_q, topk):
    g = geom.c()
    return int(lib().msa_prefill_tokens_workspace_size(ctypes.byref(g), total_units, total_q,
                                                       topk))


def msa_sparse_attn_prefill_tokens(geom: Geometry, cache: Cache, batch: Batch, q, ids, topk, out,
                                   workspace, lse=None, softmax_scale=0.0, stream=None):
    """Per-token prefill attention: ids [total_q][n_sel][topk], one list per row."""
    cache.check(geom)
    dev = cache.block_table.device
    _need(q, "q", geom.torch_dtype, 3, dev)
    _need(out, "out", geom.torch_dtype, 3, dev)
    _need(ids, "ids", torch.int32, 3, dev)
    shape = (batch.total_q, geom.num_q_heads, geom.head_dim)
    if tuple(q.shape) != shape or tuple(out.shape) != shape:
        raise ValueError(f"q and out must be {shape}")
    if tuple(ids.shape) != (batch.total_q, geom.num_sel_groups, topk):
        raise ValueError("ids must be [total_q][n_sel][topk]")
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != shape[:2]:
            raise ValueError("lse must be [total_q][H_q]")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1, dev)
    g, c, b = geom.c(), cache.c(), batch.c()
    _check(lib().msa_sparse_attn_prefill_tokens(
        ctypes.byref(g), ctypes.byref(c), ctypes.byref(b), _ptr(q), _ptr(ids), topk,
        float(softmax_scale), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _ptr(out), _ptr(lse), _stream(stream)))


def prefill_tokens(geom: Geometry, cache: Cache, batch: Batch, q, q_idx, topk, softmax_scale=0.0,
                   stream=None):
    """Index, select and attend a prefill batch with one selection per new token."""
    dev = q.device
    Q = batch.total_q
    scores = torch.empty((Q, geom.num_sel_groups, cache.max_blocks), dtype=torch.float32,
                         device=dev)
    ids = torch.empty((Q, geom.num_sel_groups, topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws = workspace(msa_prefill_tokens_workspace_size(geom, batch.total_units, Q, topk), dev)
    msa_index_scores_prefill_tokens(geom, cache, batch, q_idx, scores, stream)
    msa_select_topk_blocks(scores, topk, ids, stream)
    msa_sparse_attn_prefill_tokens(geom, cache, batch, q, ids, topk, out, ws, lse, softmax_scale,
                                   stream)
    return dict(scores=scores, ids=ids, out=out, lse=lse)


def _host_int32(t, name, ndim):
    """A C-contiguous int32 host copy of an integer tensor or array of `ndim`
    dimensions; values outside int32 are refused rather than wrapped."""
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    if a.ndim != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {a.shape}")
    if a.dtype != np.int32:
        if not np.issubdtype(a.dtype, np.integer):
            raise ValueError(f"{name} must hold integers, got {a.dtype}")
        if a.size and (a.min() < -2**31 or a.max() > 2**31 - 1):
            raise ValueError(f"{name} holds values outside int32")
    return np.ascontiguousarray(a, dtype=np.int32)


def msa_validate_block_table(block_table, seq_lens, num_phys_blocks):
    """Host check of a block table (debugging aid): raises MsaError naming the first
    entry that is not a physical block. Tensors may live on any device."""
    bt = _host_int32(block_table, "block_table", 2)
    sl = _host_int32(seq_lens, "seq_lens", 1)
    if sl.shape[0] != bt.shape[0]:
        raise ValueError(f"seq_lens has {sl.shape[0]} entries for {bt.shape[0]} table rows")
    _check(lib().msa_validate_block_table(bt.ctypes.data, sl.ctypes.data, bt.shape[0],
                                          bt.shape[1], int(num_phys_blocks)))


def msa_validate_ids(ids, max_blocks_per_seq):
    """Host check of id lists [rows][n_sel][topk] (debugging aid): raises MsaError
    naming the first list with an out-of-range or repeated entry."""
    a = _host_int32(ids, "ids", 3)
    _check(lib().msa_validate_ids(a.ctypes.data if a.size else None, a.shape[0], a.shape[1],
                                  a.shape[2], int(max_blocks_per_seq)))


def workspace(nbytes, device):
    """A 256-byte aligned uint8 device buffer of at least nbytes."""
    raw = torch.empty(max(1, nbytes) + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + max(1, nbytes)]


# ----------------------------------------------------------------------------
# whole-path helpers (allocate outputs, call the four entry points in order)
# ----------------------------------------------------------------------------

def prefill(geom: Geometry, cache: Cache, batch: Batch, q, q_idx, topk, softmax_scale=0.0,
            stream=None, staged=False):
    """Index, select and attend for a prefill batch. Returns dict of device tensors.
    staged: attention through msa_sparse_attn_prefill_staged (own workspace)."""
    dev = q.device
    U = batch.total_units
    scores = torch.empty((U, geom.num_sel_groups, cache.max_blocks), dtype=torch.float32,
                         device=dev)
    ids = torch.empty((U, geom.num_sel_groups, topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    msa_index_scores(geom, cache, batch, q_idx, scores, stream)
    msa_select_topk_blocks(scores, topk, ids, stream)
    if staged:
        ws = workspace(msa_prefill_workspace_size(geom, cache, U, topk), dev)
        msa_sparse_attn_prefill_staged(geom, cache, batch, q, ids, topk, out, ws, lse,
                                       softmax_scale, stream)
    else:
        msa_sparse_attn_prefill(geom, cache, batch, q, ids, topk, out, lse, softmax_scale,
                                stream)
    return dict(scores=scores, ids=ids, out=out, lse=lse)


def decode(geom: Geometry, cache: Cache, q, q_idx, topk, num_splits=0, softmax_scale=0.0,
           stream=None, ws=None):
    """Index, select and attend for one decode step. Returns dict of device tensors."""
    dev = q.device
    B = cache.num_seqs
    scores = torch.empty((B, geom.num_sel_groups, cache.max_blocks), dtype=torch.float32,
                         device=dev)
    ids = torch.empty((B, geom.num_sel_groups, topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(msa_decode_workspace_size(geom, B, topk, num_splits), dev)
    msa_index_scores(geom, cache, None, q_idx, scores, stream)
    msa_select_topk_blocks(scores, topk, ids, stream)
    msa_sparse_attn_decode(geom, cache, q, ids, topk, out, ws, lse, num_splits, softmax_scale,
                           stream)
    return dict(scores=scores, ids=ids, out=out, lse=lse)
