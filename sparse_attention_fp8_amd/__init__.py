"""Python binding of libdsa.so, the HIP implementation of the DeepSeek Sparse
Attention (DSA) hot path for MI355X (gfx950).

Every function here only marshals arguments (torch tensors -> device pointers,
the current HIP stream) into the C ABI declared in ``include/dsa.h``; all the
computation runs in the library's kernels.  Importing this package loads the
library and raises if it is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "LIB_PATH", "lib", "Dims", "PRODUCTION_DIMS", "rows_struct", "dims_struct",
    "indexer_scores", "topk", "topk_workspace_size", "sparse_mla_attn", "forward", "forward_noalloc",
    "forward_workspace_size", "check_index_domain",
    "sparse_mla_attn_workspace_size", "project_append", "project_append_workspace_size",
    "pages_struct", "indexer_scores_paged", "sparse_mla_attn_paged", "forward_paged",
    "project_append_paged", "indexer_loss", "indexer_loss_workspace_size", "indexer_backward",
    "indexer_backward_workspace_size", "indexer_backward_dense_workspace_size",
    "mha_prefill", "mha_prefill_workspace_size",
    "DSAError", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_OK, DSA_E_INVALID, DSA_E_UNSUPPORTED, DSA_E_WORKSPACE, DSA_E_HIP = range(5)
DSA_F32, DSA_BF16, DSA_FP8_E4M3FN = range(3)

EXPORTED_SYMBOLS = [
    "dsa_indexer_scores", "dsa_topk_workspace_size", "dsa_topk",
    "dsa_sparse_mla_attn_workspace_size",
    "dsa_sparse_mla_attn", "dsa_forward_workspace_size", "dsa_forward",
    "dsa_project_append_workspace_size", "dsa_project_append", "dsa_indexer_scores_paged",
    "dsa_sparse_mla_attn_paged", "dsa_forward_paged", "dsa_project_append_paged",
    "dsa_indexer_loss_workspace_size", "dsa_indexer_loss", "dsa_indexer_backward",
    "dsa_indexer_backward_workspace_size", "dsa_indexer_backward_dense_workspace_size",
    "dsa_indexer_loss_dense_workspace_size", "dsa_indexer_loss_dense", "dsa_indexer_backward_dense",
    "dsa_mha_prefill_workspace_size", "dsa_mha_prefill",
    "dsa_forward_noalloc", "dsa_check_index_domain", "dsa_status_string", "dsa_last_error",
    "dsa_api_version",
]


class DSAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


class _Rows(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("max_pos", ctypes.c_int32),
                ("row_seq", ctypes.c_void_p), ("row_pos", ctypes.c_void_p)]


class _Dims(ctypes.Structure):
    _fields_ = [("n_idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("qk_dim", ctypes.c_int32),
                ("v_dim", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("idx_dtype", ctypes.c_int32), ("attn_dtype", ctypes.c_int32)]


class _Pages(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("block_table", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python sparse_attention_fp8_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    R, D = ctypes.POINTER(_Rows), ctypes.POINTER(_Dims)
    L.dsa_indexer_scores.argtypes = [R, D, vp, vp, vp, vp, vp, vp, i64, vp]
    L.dsa_topk_workspace_size.argtypes = [R, i32]
    L.dsa_topk_workspace_size.restype = sz
    L.dsa_topk.argtypes = [R, i32, vp, i64, vp, vp, sz, vp]
    L.dsa_sparse_mla_attn_workspace_size.argtypes = [R, D]
    L.dsa_sparse_mla_attn_workspace_size.restype = sz
    L.dsa_sparse_mla_attn.argtypes = [R, D, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    L.dsa_forward_workspace_size.argtypes = [R, D, i32]
    L.dsa_forward_workspace_size.restype = sz
    L.dsa_forward.argtypes = [R, D, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, i32, vp, sz, vp]
    L.dsa_forward_noalloc.argtypes = [R, D, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, i32, vp]
    L.dsa_project_append_workspace_size.argtypes = [R, i32]
    L.dsa_project_append_workspace_size.restype = sz
    L.dsa_project_append.argtypes = [R, D, i32] + [vp] * 12 + [sz, vp]
    PG = ctypes.POINTER(_Pages)
    L.dsa_indexer_scores_paged.argtypes = [R, D, PG, vp, vp, vp, vp, vp, vp, i64, vp]
    L.dsa_sparse_mla_attn_paged.argtypes = [R, D, PG, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    L.dsa_forward_paged.argtypes = [R, D, PG, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, i32,
                                    vp, sz, vp]
    L.dsa_project_append_paged.argtypes = [R, D, PG, i32] + [vp] * 12 + [sz, vp]
    L.dsa_indexer_loss_workspace_size.argtypes = [R, D]
    L.dsa_indexer_loss_workspace_size.restype = sz
    L.dsa_indexer_loss.argtypes = [R, D, vp, vp, vp, vp, f32, vp, i64, vp, vp, vp, sz, vp]
    L.dsa_indexer_backward_workspace_size.argtypes = [R, D, i64]
    L.dsa_indexer_backward_workspace_size.restype = sz
    L.dsa_indexer_backward.argtypes = [R, D] + [vp] * 10 + [vp, sz, vp]
    L.dsa_indexer_loss_dense_workspace_size.argtypes = [R, D]
    L.dsa_indexer_loss_dense_workspace_size.restype = sz
    L.dsa_indexer_loss_dense.argtypes = [R, D, vp, vp, f32, vp, i64, vp, vp, vp, sz, vp]
    L.dsa_indexer_backward_dense_workspace_size.argtypes = [R, D, i64]
    L.dsa_indexer_backward_dense_workspace_size.restype = sz
    L.dsa_indexer_backward_dense.argtypes = [R, D, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz,
                                             vp]
    L.dsa_mha_prefill_workspace_size.argtypes = [R, D]
    L.dsa_mha_prefill_workspace_size.restype = sz
    L.dsa_mha_prefill.argtypes = [R, D, vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    for name in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_attn", "dsa_forward",
                 "dsa_project_append", "dsa_indexer_scores_paged", "dsa_sparse_mla_attn_paged",
                 "dsa_forward_paged", "dsa_project_append_paged", "dsa_indexer_loss",
                 "dsa_indexer_backward", "dsa_mha_prefill", "dsa_indexer_loss_dense",
                 "dsa_indexer_backward_dense", "dsa_check_index_domain", "dsa_forward_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    L.dsa_check_index_domain.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_api_version.restype = ctypes.c_int32
    return L


lib = _load()


class Dims:
    """Dimension set of a DSA layer (mirrors dsa_dims)."""

    def __init__(self, n_idx_heads, idx_dim, n_heads, qk_dim, v_dim, topk, fp32: bool):
        self.n_idx_heads, self.idx_dim, self.n_heads = n_idx_heads, idx_dim, n_heads
        self.qk_dim, self.v_dim, self.topk, self.fp32 = qk_dim, v_dim, topk, fp32

    @classmethod
    def from_config(cls, cfg) -> "Dims":
        return cls(cfg.n_idx_heads, cfg.idx_dim, cfg.n_heads, cfg.qk_dim, cfg.v_dim, cfg.topk,
                   cfg.fp32)


PRODUCTION_DIMS = Dims(64, 128, 128, 576, 512, 2048, False)


def dims_struct(d: Dims) -> _Dims:
    return _Dims(d.n_idx_heads, d.idx_dim, d.n_heads, d.qk_dim, d.v_dim, d.topk,
                 DSA_F32 if d.fp32 else DSA_FP8_E4M3FN, DSA_F32 if d.fp32 else DSA_BF16)


def rows_struct(row_seq: torch.Tensor, row_pos: torch.Tensor, num_seqs: int, max_ctx: int,
                max_pos: int) -> _Rows:
    """dsa_rows for R rows.  The struct keeps references to both tensors, so their
    device memory stays alive as long as the struct does."""
    _dev(row_seq, torch.int32, "row_seq")
    _dev(row_pos, torch.int32, "row_pos")
    if row_seq.numel() != row_pos.numel():
        raise ValueError("row_seq and row_pos must have the same length")
    rs = _Rows(row_pos.numel(), num_seqs, max_ctx, max_pos, _ptr(row_seq), _ptr(row_pos))
    rs._keep = (row_seq, row_pos)
    return rs


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: Optional[torch.Tensor], dtype, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: Optional[torch.Tensor], shape, name):
    """Check a tensor's leading dims (None = any) so a mismatch fails on the host."""
    if t is None:
        return
    if t.dim() != len(shape) or any(w is not None and a != w for a, w in zip(t.shape, shape)):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


def _caches(rows: _Rows, dims: Dims, k_idx, k_scale, latent=None):
    _shape(k_idx, (rows.num_seqs, rows.max_ctx, dims.idx_dim), "k_idx")
    _shape(k_scale, (rows.num_seqs, rows.max_ctx), "k_scale")
    _shape(latent, (rows.num_seqs, rows.max_ctx, dims.qk_dim), "latent")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int):
    if status != DSA_OK:
        raise DSAError(status, lib.dsa_last_error().decode() or lib.dsa_status_string(status).decode())


def check_index_domain() -> bool:
    """True if an attention call on the current device met an index entry past its
    row's position since the last check (dsa_check_index_domain); clears the flag."""
    seen = ctypes.c_int32(0)
    _check(lib.dsa_check_index_domain(ctypes.byref(seen)))
    return bool(seen.value)


def _idx_dtype(d: Dims):
    return torch.float32 if d.fp32 else torch.uint8


def _attn_dtype(d: Dims):
    return torch.float32 if d.fp32 else torch.bfloat16


def indexer_scores(rows: _Rows, dims: Dims, q_idx, q_scale, w, k_idx, k_scale,
                   scores: Optional[torch.Tensor] = None, ld: Optional[int] = None) -> torch.Tensor:
    """dsa_indexer_scores: returns scores [R, ld] (entries s > t unspecified)."""
    _dev(q_idx, _idx_dtype(dims), "q_idx")
    _dev(k_idx, _idx_dtype(dims), "k_idx")
    _dev(w, torch.float32, "w")
    _dev(q_scale, torch.float32, "q_scale")
    _dev(k_scale, torch.float32, "k_scale")
    R = rows.num_rows
    _shape(q_idx, (R, dims.n_idx_heads, dims.idx_dim), "q_idx")
    _shape(q_scale, (R, dims.n_idx_heads), "q_scale")
    _shape(w, (R, dims.n_idx_heads), "w")
    _caches(rows, dims, k_idx, k_scale)
    if scores is None:
        ld = ld or rows.max_pos + 1
        scores = torch.empty(rows.num_rows, ld, dtype=torch.float32, device=q_idx.device)
    _dev(scores, torch.float32, "scores")
    _shape(scores, (R, None), "scores")
    ds = dims_struct(dims)
    _check(lib.dsa_indexer_scores(ctypes.byref(rows), ctypes.byref(ds), _ptr(q_idx), _ptr(q_scale),
                                  _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(scores),
                                  scores.shape[1], _stream()))
    return scores


def topk_workspace_size(rows: _Rows, k: int) -> int:
    return int(lib.dsa_topk_workspace_size(ctypes.byref(rows), int(k)))


def topk(rows: _Rows, k: int, scores: torch.Tensor,
         indices: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dsa_topk: returns indices [R, k] int32 (ascending, -1 padded)."""
    _dev(scores, torch.float32, "scores")
    if indices is None:
        indices = torch.empty(rows.num_rows, k, dtype=torch.int32, device=scores.device)
    need = topk_workspace_size(rows, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    _dev(workspace, torch.uint8, "workspace")
    _dev(indices, torch.int32, "indices")
    _shape(scores, (rows.num_rows, None), "scores")
    _shape(indices, (rows.num_rows, k), "indices")
    _check(lib.dsa_topk(ctypes.byref(rows), k, _ptr(scores), scores.shape[1], _ptr(indices),
                        _ptr(workspace), 0 if workspace is None else workspace.numel(),
                        _stream()))
    return indices


def sparse_mla_attn_workspace_size(rows: _Rows, dims: Dims) -> int:
    ds = dims_struct(dims)
    return int(lib.dsa_sparse_mla_attn_workspace_size(ctypes.byref(rows), ctypes.byref(ds)))


def sparse_mla_attn(rows: _Rows, dims: Dims, q, latent, indices, softmax_scale: float,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """dsa_sparse_mla_attn: returns (out [R,H,D_v], lse [R,H])."""
    adt = _attn_dtype(dims)
    _dev(q, adt, "q")
    _dev(latent, adt, "latent")
    _dev(indices, torch.int32, "indices")
    R = rows.num_rows
    if out is None:
        out = torch.empty(R, dims.n_heads, dims.v_dim, dtype=adt, device=q.device)
    if lse is None:
        lse = torch.empty(R, dims.n_heads, dtype=torch.float32, device=q.device)
    _dev(out, adt, "out")
    _dev(lse, torch.float32, "lse")
    _shape(q, (R, dims.n_heads, dims.qk_dim), "q")
    _shape(indices, (R, dims.topk), "indices")
    _shape(out, (R, dims.n_heads, dims.v_dim), "out")
    _shape(lse, (R, dims.n_heads), "lse")
    _caches(rows, dims, None, None, latent)
    need = sparse_mla_attn_workspace_size(rows, dims)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    ds = dims_struct(dims)
    _check(lib.dsa_sparse_mla_attn(ctypes.byref(rows), ctypes.byref(ds), _ptr(q), _ptr(latent),
                                   _ptr(indices), float(softmax_scale), _ptr(out), _ptr(lse),
                                   _ptr(workspace), ws_bytes, _stream()))
    return out, lse


def forward_workspace_size(rows: _Rows, dims: Dims, chunk_rows: int = 0) -> int:
    ds = dims_struct(dims)
    return int(lib.dsa_forward_workspace_size(ctypes.byref(rows), ctypes.byref(ds), chunk_rows))


def _forward_outputs(rows: _Rows, dims: Dims, q_idx, q_scale, w, k_idx, k_scale, q, latent,
                     out, lse, indices_out):
    """Shape / dtype checks of the dsa_forward arguments; allocates out and lse when
    not given."""
    adt = _attn_dtype(dims)
    for t, dt, name in ((q_idx, _idx_dtype(dims), "q_idx"), (k_idx, _idx_dtype(dims), "k_idx"),
                        (w, torch.float32, "w"), (q_scale, torch.float32, "q_scale"),
                        (k_scale, torch.float32, "k_scale"), (q, adt, "q"), (latent, adt, "latent")):
        _dev(t, dt, name)
    R = rows.num_rows
    if out is None:
        out = torch.empty(R, dims.n_heads, dims.v_dim, dtype=adt, device=q.device)
    if lse is None:
        lse = torch.empty(R, dims.n_heads, dtype=torch.float32, device=q.device)
    _dev(out, adt, "out")
    _dev(lse, torch.float32, "lse")
    _dev(indices_out, torch.int32, "indices_out")
    _shape(q_idx, (R, dims.n_idx_heads, dims.idx_dim), "q_idx")
    _shape(q_scale, (R, dims.n_idx_heads), "q_scale")
    _shape(w, (R, dims.n_idx_heads), "w")
    _shape(q, (R, dims.n_heads, dims.qk_dim), "q")
    _shape(out, (R, dims.n_heads, dims.v_dim), "out")
    _shape(lse, (R, dims.n_heads), "lse")
    _shape(indices_out, (R, dims.topk), "indices_out")
    _caches(rows, dims, k_idx, k_scale, latent)
    return out, lse


def forward(rows: _Rows, dims: Dims, q_idx, q_scale, w, k_idx, k_scale, q, latent,
            softmax_scale: float, out=None, lse=None, indices_out=None, chunk_rows: int = 0,
            workspace: Optional[torch.Tensor] = None):
    """dsa_forward: indexer -> top-k -> attention.  Returns (out, lse, indices_out)."""
    out, lse = _forward_outputs(rows, dims, q_idx, q_scale, w, k_idx, k_scale, q, latent, out,
                                lse, indices_out)
    need = forward_workspace_size(rows, dims, chunk_rows)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, torch.uint8, "workspace")
    ds = dims_struct(dims)
    _check(lib.dsa_forward(ctypes.byref(rows), ctypes.byref(ds), _ptr(q_idx), _ptr(q_scale),
                           _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(q), _ptr(latent),
                           float(softmax_scale), _ptr(out), _ptr(lse), _ptr(indices_out),
                           int(chunk_rows), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse, indices_out


def forward_noalloc(rows: _Rows, dims: Dims, q_idx, q_scale, w, k_idx, k_scale, q, latent,
                    softmax_scale: float, out, lse, indices_out=None, chunk_rows: int = 0):
    """dsa_forward_noalloc: dsa_forward with the library's fixed scratch.  out and
    lse must be given (nothing is allocated here either)."""
    if out is None or lse is None:
        raise ValueError("forward_noalloc writes into caller-provided out and lse")
    _forward_outputs(rows, dims, q_idx, q_scale, w, k_idx, k_scale, q, latent, out, lse,
                     indices_out)
    ds = dims_struct(dims)
    _check(lib.dsa_forward_noalloc(ctypes.byref(rows), ctypes.byref(ds), _ptr(q_idx),
                                   _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale), _ptr(q),
                                   _ptr(latent), float(softmax_scale), _ptr(out), _ptr(lse),
                                   _ptr(indices_out), int(chunk_rows), _stream()))
    return out, lse, indices_out


def project_append_workspace_size(rows: _Rows, d_model: int) -> int:
    return int(lib.dsa_project_append_workspace_size(ctypes.byref(rows), int(d_model)))


def project_append(rows: _Rows, h, w_q, w_k, w_c, w_w, k_idx, k_scale, latent,
                   q_idx=None, q_scale=None, w=None, dims: Dims = PRODUCTION_DIMS,
                   workspace: Optional[torch.Tensor] = None):
    """dsa_project_append: projections of the R tokens in h, their indexer query
    and head weights returned as (q_idx, q_scale, w); the indexer key and latent
    rows are written into the caches k_idx/k_scale/latent in place."""
    R, d_model = h.shape[0], h.shape[-1]
    _dev(h, torch.bfloat16, "h")
    for t, name in ((w_q, "w_q"), (w_k, "w_k"), (w_c, "w_c"), (w_w, "w_w")):
        _dev(t, torch.bfloat16, name)
    _shape(h, (rows.num_rows, None), "h")
    _shape(w_q, (dims.n_idx_heads * dims.idx_dim, d_model), "w_q")
    _shape(w_k, (dims.idx_dim, d_model), "w_k")
    _shape(w_c, (dims.qk_dim, d_model), "w_c")
    _shape(w_w, (dims.n_idx_heads, d_model), "w_w")
    if q_idx is None:
        q_idx = torch.empty(R, dims.n_idx_heads, dims.idx_dim, dtype=torch.uint8, device=h.device)
    if q_scale is None:
        q_scale = torch.empty(R, dims.n_idx_heads, dtype=torch.float32, device=h.device)
    if w is None:
        w = torch.empty(R, dims.n_idx_heads, dtype=torch.float32, device=h.device)
    _dev(q_idx, torch.uint8, "q_idx")
    _dev(q_scale, torch.float32, "q_scale")
    _dev(w, torch.float32, "w")
    _dev(k_idx, torch.uint8, "k_idx")
    _dev(k_scale, torch.float32, "k_scale")
    _dev(latent, torch.bfloat16, "latent")
    _shape(q_idx, (R, dims.n_idx_heads, dims.idx_dim), "q_idx")
    _shape(q_scale, (R, dims.n_idx_heads), "q_scale")
    _shape(w, (R, dims.n_idx_heads), "w")
    _caches(rows, dims, k_idx, k_scale, latent)
    need = project_append_workspace_size(rows, d_model)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=h.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    ds = dims_struct(dims)
    _check(lib.dsa_project_append(ctypes.byref(rows), ctypes.byref(ds), int(d_model), _ptr(h),
                                  _ptr(w_q), _ptr(w_k), _ptr(w_c), _ptr(w_w), _ptr(q_idx),
                                  _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale),
                                  _ptr(latent), _ptr(workspace), ws_bytes, _stream()))
    return q_idx, q_scale, w


# ---------------------------------------------------------------- paged caches

def pages_struct(block_table: torch.Tensor, page_size: int, num_pages: int) -> _Pages:
    """dsa_pages for a device block table [B, pages_per_seq] int32 (kept alive by
    the struct)."""
    _dev(block_table, torch.int32, "block_table")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, pages_per_seq]")
    ps = _Pages(int(page_size), block_table.shape[1], int(num_pages), _ptr(block_table))
    ps._keep = block_table
    return ps


def _pools(pages: _Pages, dims: Dims, k_pool=None, k_scale_pool=None, latent_pool=None):
    P, n = pages.page_size, pages.num_pages
    _shape(k_pool, (n, P, dims.idx_dim), "k_pool")
    _shape(k_scale_pool, (n, P), "k_scale_pool")
    _shape(latent_pool, (n, P, dims.qk_dim), "latent_pool")


def indexer_scores_paged(rows: _Rows, dims: Dims, pages: _Pages, q_idx, q_scale, w, k_pool,
                         k_scale_pool, scores: Optional[torch.Tensor] = None,
                         ld: Optional[int] = None) -> torch.Tensor:
    """dsa_indexer_scores_paged: scores [R, ld] from paged key / scale pools."""
    for t, dt, name in ((q_idx, torch.uint8, "q_idx"), (k_pool, torch.uint8, "k_pool"),
                        (w, torch.float32, "w"), (q_scale, torch.float32, "q_scale"),
                        (k_scale_pool, torch.float32, "k_scale_pool")):
        _dev(t, dt, name)
    R = rows.num_rows
    _shape(q_idx, (R, dims.n_idx_heads, dims.idx_dim), "q_idx")
    _shape(q_scale, (R, dims.n_idx_heads), "q_scale")
    _shape(w, (R, dims.n_idx_heads), "w")
    _pools(pages, dims, k_pool, k_scale_pool)
    if scores is None:
        ld = ld or rows.max_pos + 1
        scores = torch.empty(R, ld, dtype=torch.float32, device=q_idx.device)
    _dev(scores, torch.float32, "scores")
    _shape(scores, (R, None), "scores")
    ds = dims_struct(dims)
    _check(lib.dsa_indexer_scores_paged(ctypes.byref(rows), ctypes.byref(ds), ctypes.byref(pages),
                                        _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_pool),
                                        _ptr(k_scale_pool), _ptr(scores), scores.shape[1],
                                        _stream()))
    return scores


def sparse_mla_attn_paged(rows: _Rows, dims: Dims, pages: _Pages, q, latent_pool, indices,
                          softmax_scale: float, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None):
    """dsa_sparse_mla_attn_paged: (out, lse) from a paged latent pool."""
    _dev(q, torch.bfloat16, "q")
    _dev(latent_pool, torch.bfloat16, "latent_pool")
    _dev(indices, torch.int32, "indices")
    R = rows.num_rows
    if out is None:
        out = torch.empty(R, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(R, dims.n_heads, dtype=torch.float32, device=q.device)
    _dev(out, torch.bfloat16, "out")
    _dev(lse, torch.float32, "lse")
    _shape(q, (R, dims.n_heads, dims.qk_dim), "q")
    _shape(indices, (R, dims.topk), "indices")
    _shape(out, (R, dims.n_heads, dims.v_dim), "out")
    _pools(pages, dims, latent_pool=latent_pool)
    need = sparse_mla_attn_workspace_size(rows, dims)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    ds = dims_struct(dims)
    _check(lib.dsa_sparse_mla_attn_paged(ctypes.byref(rows), ctypes.byref(ds), ctypes.byref(pages),
                                         _ptr(q), _ptr(latent_pool), _ptr(indices),
                                         float(softmax_scale), _ptr(out), _ptr(lse),
                                         _ptr(workspace), ws_bytes, _stream()))
    return out, lse


def forward_paged(rows: _Rows, dims: Dims, pages: _Pages, q_idx, q_scale, w, k_pool,
                  k_scale_pool, q, latent_pool, softmax_scale: float, out=None, lse=None,
                  indices_out=None, chunk_rows: int = 0,
                  workspace: Optional[torch.Tensor] = None):
    """dsa_forward_paged: the whole path over paged caches; (out, lse, indices_out)."""
    for t, dt, name in ((q_idx, torch.uint8, "q_idx"), (k_pool, torch.uint8, "k_pool"),
                        (w, torch.float32, "w"), (q_scale, torch.float32, "q_scale"),
                        (k_scale_pool, torch.float32, "k_scale_pool"), (q, torch.bfloat16, "q"),
                        (latent_pool, torch.bfloat16, "latent_pool")):
        _dev(t, dt, name)
    R = rows.num_rows
    if out is None:
        out = torch.empty(R, dims.n_heads, dims.v_dim, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(R, dims.n_heads, dtype=torch.float32, device=q.device)
    _dev(out, torch.bfloat16, "out")
    _dev(lse, torch.float32, "lse")
    _dev(indices_out, torch.int32, "indices_out")
    _shape(q_idx, (R, dims.n_idx_heads, dims.idx_dim), "q_idx")
    _shape(q_scale, (R, dims.n_idx_heads), "q_scale")
    _shape(w, (R, dims.n_idx_heads), "w")
    _shape(q, (R, dims.n_heads, dims.qk_dim), "q")
    _shape(out, (R, dims.n_heads, dims.v_dim), "out")
    _shape(indices_out, (R, dims.topk), "indices_out")
    _pools(pages, dims, k_pool, k_scale_pool, latent_pool)
    need = forward_workspace_size(rows, dims, chunk_rows)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, torch.uint8, "workspace")
    ds = dims_struct(dims)
    _check(lib.dsa_forward_paged(ctypes.byref(rows), ctypes.byref(ds), ctypes.byref(pages),
                                 _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_pool),
                                 _ptr(k_scale_pool), _ptr(q), _ptr(latent_pool),
                                 float(softmax_scale), _ptr(out), _ptr(lse), _ptr(indices_out),
                                 int(chunk_rows), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse, indices_out


def project_append_paged(rows: _Rows, pages: _Pages, h, w_q, w_k, w_c, w_w, k_pool,
                         k_scale_pool, latent_pool, q_idx=None, q_scale=None, w=None,
                         dims: Dims = PRODUCTION_DIMS, workspace: Optional[torch.Tensor] = None):
    """dsa_project_append_paged: as project_append, appending into paged pools."""
    R, d_model = h.shape[0], h.shape[-1]
    _dev(h, torch.bfloat16, "h")
    for t, name in ((w_q, "w_q"), (w_k, "w_k"), (w_c, "w_c"), (w_w, "w_w")):
        _dev(t, torch.bfloat16, name)
    _shape(h, (R, None), "h")
    _shape(w_q, (dims.n_idx_heads * dims.idx_dim, d_model), "w_q")
    _shape(w_k, (dims.idx_dim, d_model), "w_k")
    _shape(w_c, (dims.qk_dim, d_model), "w_c")
    _shape(w_w, (dims.n_idx_heads, d_model), "w_w")
    if q_idx is None:
        q_idx = torch.empty(R, dims.n_idx_heads, dims.idx_dim, dtype=torch.uint8, device=h.device)
    if q_scale is None:
        q_scale = torch.empty(R, dims.n_idx_heads, dtype=torch.float32, device=h.device)
    if w is None:
        w = torch.empty(R, dims.n_idx_heads, dtype=torch.float32, device=h.device)
    _dev(k_pool, torch.uint8, "k_pool")
    _dev(k_scale_pool, torch.float32, "k_scale_pool")
    _dev(latent_pool, torch.bfloat16, "latent_pool")
    _pools(pages, dims, k_pool, k_scale_pool, latent_pool)
    need = project_append_workspace_size(rows, d_model)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=h.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    ds = dims_struct(dims)
    _check(lib.dsa_project_append_paged(ctypes.byref(rows), ctypes.byref(ds), ctypes.byref(pages),
                                        int(d_model), _ptr(h), _ptr(w_q), _ptr(w_k), _ptr(w_c),
                                        _ptr(w_w), _ptr(q_idx), _ptr(q_scale), _ptr(w),
                                        _ptr(k_pool), _ptr(k_scale_pool), _ptr(latent_pool),
                                        _ptr(workspace), ws_bytes, _stream()))
    return q_idx, q_scale, w


# ---------------------------------------------------------------- indexer training loss

def indexer_loss_workspace_size(rows: _Rows, dims: Dims = PRODUCTION_DIMS) -> int:
    ds = dims_struct(dims)
    return int(lib.dsa_indexer_loss_workspace_size(ctypes.byref(rows), ctypes.byref(ds)))


def indexer_loss(rows: _Rows, q, latent, indices, lse, softmax_scale: float, scores,
                 dims: Dims = PRODUCTION_DIMS, loss=None, dscores=None,
                 workspace: Optional[torch.Tensor] = None):
    """dsa_indexer_loss: (loss [R], dscores [R, k]) of the sparse-stage KL."""
    R = rows.num_rows
    _dev(q, torch.bfloat16, "q")
    _dev(latent, torch.bfloat16, "latent")
    _dev(indices, torch.int32, "indices")
    _dev(lse, torch.float32, "lse")
    _dev(scores, torch.float32, "scores")
    _shape(q, (R, dims.n_heads, dims.qk_dim), "q")
    _shape(indices, (R, dims.topk), "indices")
    _shape(lse, (R, dims.n_heads), "lse")
    _shape(scores, (R, None), "scores")
    _caches(rows, dims, None, None, latent)
    if loss is None:
        loss = torch.empty(R, dtype=torch.float32, device=q.device)
    if dscores is None:
        dscores = torch.empty(R, dims.topk, dtype=torch.float32, device=q.device)
    _dev(loss, torch.float32, "loss")
    _dev(dscores, torch.float32, "dscores")
    need = indexer_loss_workspace_size(rows, dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ds = dims_struct(dims)
    _check(lib.dsa_indexer_loss(ctypes.byref(rows), ctypes.byref(ds), _ptr(q), _ptr(latent),
                                _ptr(indices), _ptr(lse), float(softmax_scale), _ptr(scores),
                                scores.shape[1], _ptr(loss), _ptr(dscores), _ptr(workspace),
                                workspace.numel(), _stream()))
    return loss, dscores


def indexer_loss_dense_workspace_size(rows: _Rows, dims: Dims = PRODUCTION_DIMS) -> int:
    ds = dims_struct(dims)
    return int(lib.dsa_indexer_loss_dense_workspace_size(ctypes.byref(rows), ctypes.byref(ds)))


def indexer_loss_dense(rows: _Rows, q, latent, softmax_scale: float, scores,
                       dims: Dims = PRODUCTION_DIMS, loss=None, dscores=None,
                       workspace: Optional[torch.Tensor] = None):
    """dsa_indexer_loss_dense: (loss [R], dscores [R, ld]) of the dense warm-up KL."""
    R = rows.num_rows
    _dev(q, torch.bfloat16, "q")
    _dev(latent, torch.bfloat16, "latent")
    _dev(scores, torch.float32, "scores")
    _shape(q, (R, dims.n_heads, dims.qk_dim), "q")
    _shape(scores, (R, None), "scores")
    _caches(rows, dims, None, None, latent)
    if loss is None:
        loss = torch.empty(R, dtype=torch.float32, device=q.device)
    if dscores is None:
        dscores = torch.empty_like(scores)
    _dev(loss, torch.float32, "loss")
    _dev(dscores, torch.float32, "dscores")
    _shape(dscores, tuple(scores.shape), "dscores")
    need = indexer_loss_dense_workspace_size(rows, dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ds = dims_struct(dims)
    _check(lib.dsa_indexer_loss_dense(ctypes.byref(rows), ctypes.byref(ds), _ptr(q), _ptr(latent),
                                      float(softmax_scale), _ptr(scores), scores.shape[1],
                                      _ptr(loss), _ptr(dscores), _ptr(workspace),
                                      workspace.numel(), _stream()))
    return loss, dscores


def indexer_backward_workspace_size(rows: _Rows, dims: Dims = PRODUCTION_DIMS,
                                    shared_keys: int = -1) -> int:
    ds = dims_struct(dims)
    return int(lib.dsa_indexer_backward_workspace_size(ctypes.byref(rows), ctypes.byref(ds),
                                                       int(shared_keys)))


def indexer_backward_dense_workspace_size(rows: _Rows, dims: Dims = PRODUCTION_DIMS,
                                          shared_keys: int = -1) -> int:
    ds = dims_struct(dims)
    return int(lib.dsa_indexer_backward_dense_workspace_size(ctypes.byref(rows),
                                                             ctypes.byref(ds), int(shared_keys)))


def _bwd_workspace(workspace, need, device):
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _dev(workspace, torch.uint8, "workspace")
    return workspace


def indexer_backward(rows: _Rows, q_idx, q_scale, w, k_idx, k_scale, indices, dscores, dq, dw,
                     dk, dims: Dims = PRODUCTION_DIMS, workspace: Optional[torch.Tensor] = None):
    """dsa_indexer_backward: adds the gradients into dq [R,H_I,d_I], dw [R,H_I] and
    dk [B,N,d_I] (fp32, zeroed by the caller).  Without a workspace, one of the full
    size (room for every key the call could select twice) is allocated."""
    R = rows.num_rows
    for t, dt, name in ((q_idx, torch.uint8, "q_idx"), (q_scale, torch.float32, "q_scale"),
                        (w, torch.float32, "w"), (k_idx, torch.uint8, "k_idx"),
                        (k_scale, torch.float32, "k_scale"), (indices, torch.int32, "indices"),
                        (dscores, torch.float32, "dscores"), (dq, torch.float32, "dq"),
                        (dw, torch.float32, "dw"), (dk, torch.float32, "dk")):
        _dev(t, dt, name)
    _shape(q_idx, (R, dims.n_idx_heads, dims.idx_dim), "q_idx")
    _shape(dq, (R, dims.n_idx_heads, dims.idx_dim), "dq")
    _shape(dw, (R, dims.n_idx_heads), "dw")
    _shape(indices, (R, dims.topk), "indices")
    _shape(dscores, (R, dims.topk), "dscores")
    _caches(rows, dims, k_idx, k_scale)
    _shape(dk, (rows.num_seqs, rows.max_ctx, dims.idx_dim), "dk")
    workspace = _bwd_workspace(workspace, indexer_backward_workspace_size(rows, dims), dq.device)
    ds = dims_struct(dims)
    _check(lib.dsa_indexer_backward(ctypes.byref(rows), ctypes.byref(ds), _ptr(q_idx),
                                    _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale),
                                    _ptr(indices), _ptr(dscores), _ptr(dq), _ptr(dw), _ptr(dk),
                                    _ptr(workspace), workspace.numel(), _stream()))
    return dq, dw, dk


def indexer_backward_dense(rows: _Rows, q_idx, q_scale, w, k_idx, k_scale, dscores, dq, dw, dk,
                           dims: Dims = PRODUCTION_DIMS,
                           workspace: Optional[torch.Tensor] = None):
    """dsa_indexer_backward_dense: the dense warm-up loss's dscores [R, ld] (by position)
    into dq, dw and dk (fp32, accumulated; zeroed by the caller).  Without a
    workspace, one of the full size is allocated."""
    R = rows.num_rows
    for t, dt, name in ((q_idx, torch.uint8, "q_idx"), (q_scale, torch.float32, "q_scale"),
                        (w, torch.float32, "w"), (k_idx, torch.uint8, "k_idx"),
                        (k_scale, torch.float32, "k_scale"), (dscores, torch.float32, "dscores"),
                        (dq, torch.float32, "dq"), (dw, torch.float32, "dw"),
                        (dk, torch.float32, "dk")):
        _dev(t, dt, name)
    _shape(q_idx, (R, dims.n_idx_heads, dims.idx_dim), "q_idx")
    _shape(dq, (R, dims.n_idx_heads, dims.idx_dim), "dq")
    _shape(dw, (R, dims.n_idx_heads), "dw")
    _shape(dscores, (R, None), "dscores")
    _caches(rows, dims, k_idx, k_scale)
    _shape(dk, (rows.num_seqs, rows.max_ctx, dims.idx_dim), "dk")
    workspace = _bwd_workspace(workspace, indexer_backward_dense_workspace_size(rows, dims),
                               dq.device)
    ds = dims_struct(dims)
    _check(lib.dsa_indexer_backward_dense(ctypes.byref(rows), ctypes.byref(ds), _ptr(q_idx),
                                          _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale),
                                          _ptr(dscores), dscores.shape[1], _ptr(dq), _ptr(dw),
                                          _ptr(dk), _ptr(workspace), workspace.numel(),
                                          _stream()))
    return dq, dw, dk


# ---------------------------------------------------------------- masked MHA mode

def mha_prefill_workspace_size(rows: _Rows, dims: Dims = PRODUCTION_DIMS) -> int:
    ds = dims_struct(dims)
    return int(lib.dsa_mha_prefill_workspace_size(ctypes.byref(rows), ctypes.byref(ds)))


def mha_prefill(rows: _Rows, q, latent, w_uk, w_uv, indices, softmax_scale: float,
                dims: Dims = PRODUCTION_DIMS, out=None, lse=None,
                workspace: Optional[torch.Tensor] = None):
    """dsa_mha_prefill: (out [R, H, 128] bf16, lse [R, H]) of the masked MHA mode."""
    R = rows.num_rows
    for t, name in ((q, "q"), (latent, "latent"), (w_uk, "w_uk"), (w_uv, "w_uv")):
        _dev(t, torch.bfloat16, name)
    _dev(indices, torch.int32, "indices")
    _shape(q, (R, dims.n_heads, 192), "q")
    _shape(w_uk, (dims.n_heads, 128, dims.v_dim), "w_uk")
    _shape(w_uv, (dims.n_heads, 128, dims.v_dim), "w_uv")
    _shape(indices, (R, dims.topk), "indices")
    _caches(rows, dims, None, None, latent)
    if out is None:
        out = torch.empty(R, dims.n_heads, 128, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(R, dims.n_heads, dtype=torch.float32, device=q.device)
    _dev(out, torch.bfloat16, "out")
    _dev(lse, torch.float32, "lse")
    need = mha_prefill_workspace_size(rows, dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ds = dims_struct(dims)
    _check(lib.dsa_mha_prefill(ctypes.byref(rows), ctypes.byref(ds), _ptr(q), _ptr(latent),
                               _ptr(w_uk), _ptr(w_uv), _ptr(indices), float(softmax_scale),
                               _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                               _stream()))
    return out, lse
