"""ctypes binding of libmla_verify.so: argument marshalling only.

Every step of the verify path runs in the library's gfx950 kernels; this module
checks tensor dtypes, devices and shapes, fills the descriptor and passes raw
device pointers and the current HIP stream. The library is loaded from the
package's lib/ directory; calls fail loudly if it was not built.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmla_verify.so")

HEAD_DIM_QK = 576
HEAD_DIM_V = 512
DEVERR_BAD_PARENT = 1
DEVERR_SEQ_LEN = 2
DEVERR_SLOT_RANGE = 4
DEVERR_INDEX_RANGE = 8

STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_UNSUPPORTED",
          -4: "MLA_ERR_WORKSPACE", -5: "MLA_ERR_ALIGN", -6: "MLA_ERR_HIP", -7: "MLA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_VERIFY_NOALLOC_SCRATCH_BYTES


class MlaVerifyDesc(ctypes.Structure):
    """Mirror of mla_verify_desc (include/mla_verify.h)."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_nodes", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("nsplit", ctypes.c_int32),
        ("num_kv_slots", ctypes.c_int64),
        ("kv_row_stride", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
    ]


class MlaSparseDesc(ctypes.Structure):
    """Mirror of mla_sparse_desc (include/mla_spec_ops.h)."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("nsplit", ctypes.c_int32),
        ("num_kv_slots", ctypes.c_int64),
        ("kv_row_stride", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
    ]


class MlaIndexerDesc(ctypes.Structure):
    """Mirror of mla_indexer_desc (include/mla_spec_ops.h)."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
    ]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


_LIB = None


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load the built library (once). Raises if it is missing: there is no
    fallback path."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with python -m speculative_decoding_mla_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.mla_verify_workspace_bytes.argtypes = [ctypes.POINTER(MlaVerifyDesc)]
        lib.mla_verify_workspace_bytes.restype = sz
        lib.mla_build_tree_mask.argtypes = [vp, vp, i32, i32, vp, vp]
        lib.mla_build_tree_mask.restype = ctypes.c_int
        lib.mla_verify_attention.argtypes = [ctypes.POINTER(MlaVerifyDesc), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_verify_attention.restype = ctypes.c_int
        lib.mla_verify_partial.argtypes = [ctypes.POINTER(MlaVerifyDesc), vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_verify_partial.restype = ctypes.c_int
        lib.mla_verify_combine.argtypes = [ctypes.POINTER(MlaVerifyDesc), vp, vp, vp, sz, vp]
        lib.mla_verify_combine.restype = ctypes.c_int
        lib.mla_verify_attention_noalloc.argtypes = [ctypes.POINTER(MlaVerifyDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                                     vp]
        lib.mla_verify_attention_noalloc.restype = ctypes.c_int
        lib.mla_status_string.argtypes = [ctypes.c_int]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_verify_abi_version.argtypes = []
        lib.mla_verify_abi_version.restype = i32
        i64 = ctypes.c_int64
        lib.mla_sparse_decode_workspace_bytes.argtypes = [ctypes.POINTER(MlaSparseDesc)]
        lib.mla_sparse_decode_workspace_bytes.restype = sz
        lib.mla_sparse_decode.argtypes = [ctypes.POINTER(MlaSparseDesc), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.mla_sparse_decode.restype = ctypes.c_int
        lib.mla_kv_append.argtypes = [vp, i64, i64, vp, vp, i32, vp, vp]
        lib.mla_kv_append.restype = ctypes.c_int
        lib.mla_tree_accept.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
        lib.mla_tree_accept.restype = ctypes.c_int
        lib.mla_commit_accepted.argtypes = [vp, i32, vp, i32, i32, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp]
        lib.mla_commit_accepted.restype = ctypes.c_int
        lib.mla_accept_commit.argtypes = [vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp,
                                          vp, vp]
        lib.mla_accept_commit.restype = ctypes.c_int
        lib.mla_window_map.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp, vp]
        lib.mla_window_map.restype = ctypes.c_int
        lib.mla_indexer_logits.argtypes = [ctypes.POINTER(MlaIndexerDesc), vp, vp, vp, vp, vp, vp, vp, vp]
        lib.mla_indexer_logits.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def make_desc(*, batch: int, num_nodes: int, num_heads: int, page_size: int, max_pages: int,
              nsplit: int, num_kv_slots: int, kv_row_stride: int = HEAD_DIM_QK,
              sm_scale: float = 1.0 / math.sqrt(192.0), head_dim_qk: int = HEAD_DIM_QK,
              head_dim_v: int = HEAD_DIM_V) -> MlaVerifyDesc:
    return MlaVerifyDesc(batch, num_nodes, num_heads, head_dim_qk, head_dim_v, page_size, max_pages,
                         nsplit, num_kv_slots, kv_row_stride, sm_scale)


def workspace_bytes(desc: MlaVerifyDesc) -> int:
    return int(load_library().mla_verify_workspace_bytes(ctypes.byref(desc)))


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else int(t.data_ptr())


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def desc_for(q: torch.Tensor, kv_cache: torch.Tensor, page_table: torch.Tensor, *, page_size: int,
             nsplit: int, sm_scale: float) -> MlaVerifyDesc:
    """Descriptor from tensor shapes: q [B,T,H,576], kv_cache [slots, stride>=576],
    page_table [B, max_pages]."""
    b, t, h, d = q.shape
    return make_desc(batch=b, num_nodes=t, num_heads=h, page_size=page_size, max_pages=page_table.shape[1],
                     nsplit=nsplit, num_kv_slots=kv_cache.shape[0], kv_row_stride=kv_cache.stride(0),
                     sm_scale=sm_scale, head_dim_qk=d)


def verify_attention(q: torch.Tensor, kv_cache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                     tree_parent: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, workspace: torch.Tensor,
                     *, page_size: int, nsplit: int, sm_scale: float, stream=None) -> None:
    """Enqueue mla_verify_attention on `stream` (default: torch's current stream).
    Writes out (bf16 [B,T,H,512]) and lse (fp32 [B,T,H]) in place."""
    lib = load_library()
    b, t, h, d = q.shape
    _need(q.dtype == torch.bfloat16 and q.is_contiguous(), "q must be contiguous bf16 [B,T,H,576]")
    _need(kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 2 and kv_cache.stride(1) == 1,
          "kv_cache must be bf16 [slots, stride] with unit inner stride")
    _need(page_table.dtype == torch.int32 and page_table.is_contiguous() and page_table.shape[0] == b,
          "page_table must be contiguous int32 [B, max_pages]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_contiguous() and seq_lens.numel() == b,
          "seq_lens must be int32 [B]")
    _need(tree_parent.dtype == torch.int32 and tree_parent.is_contiguous() and tuple(tree_parent.shape) == (b, t),
          "tree_parent must be contiguous int32 [B,T]")
    _need(out.dtype == torch.bfloat16 and out.is_contiguous() and tuple(out.shape) == (b, t, h, HEAD_DIM_V),
          "out must be contiguous bf16 [B,T,H,512]")
    _need(lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (b, t, h),
          "lse must be contiguous fp32 [B,T,H]")
    tensors = (q, kv_cache, page_table, seq_lens, tree_parent, out, lse, workspace)
    _need(all(x.is_cuda for x in tensors), "all tensors must be on the GPU")
    desc = desc_for(q, kv_cache, page_table, page_size=page_size, nsplit=nsplit, sm_scale=sm_scale)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.mla_verify_attention(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(page_table), _ptr(seq_lens),
                                  _ptr(tree_parent), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                  _stream_handle(stream))
    if st != 0:
        raise MlaError("mla_verify_attention", st)


def verify_attention_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, page_table: torch.Tensor,
                             seq_lens: torch.Tensor, tree_parent: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                             dev_err: torch.Tensor | None = None, *, page_size: int, nsplit: int, sm_scale: float,
                             stream=None) -> None:
    """Enqueue mla_verify_attention_noalloc: the same call with no workspace (the
    library's static per-GPU scratch holds the split partials). dev_err: an
    optional int32 tensor whose first word receives the sticky device error bits."""
    lib = load_library()
    b, t, h, d = q.shape
    _need(q.dtype == torch.bfloat16 and q.is_contiguous(), "q must be contiguous bf16 [B,T,H,576]")
    _need(kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 2 and kv_cache.stride(1) == 1,
          "kv_cache must be bf16 [slots, stride] with unit inner stride")
    _need(page_table.dtype == torch.int32 and page_table.is_contiguous() and page_table.shape[0] == b,
          "page_table must be contiguous int32 [B, max_pages]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_contiguous() and seq_lens.numel() == b,
          "seq_lens must be int32 [B]")
    _need(tree_parent.dtype == torch.int32 and tree_parent.is_contiguous() and tuple(tree_parent.shape) == (b, t),
          "tree_parent must be contiguous int32 [B,T]")
    _need(out.dtype == torch.bfloat16 and out.is_contiguous() and tuple(out.shape) == (b, t, h, HEAD_DIM_V),
          "out must be contiguous bf16 [B,T,H,512]")
    _need(lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (b, t, h),
          "lse must be contiguous fp32 [B,T,H]")
    _need(dev_err is None or (dev_err.dtype == torch.int32 and dev_err.is_cuda), "dev_err must be int32 on the GPU")
    _need(all(x.is_cuda for x in (q, kv_cache, page_table, seq_lens, tree_parent, out, lse)),
          "all tensors must be on the GPU")
    desc = desc_for(q, kv_cache, page_table, page_size=page_size, nsplit=nsplit, sm_scale=sm_scale)
    st = lib.mla_verify_attention_noalloc(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(page_table),
                                          _ptr(seq_lens), _ptr(tree_parent), _ptr(out), _ptr(lse), _ptr(dev_err),
                                          _stream_handle(stream))
    if st != 0:
        raise MlaError("mla_verify_attention_noalloc", st)


def verify_partial(desc: MlaVerifyDesc, q, kv_cache, page_table, seq_lens, tree_parent, workspace,
                   stream=None) -> None:
    """Enqueue only the split-partial stage (mla_verify_partial) for a prepared
    descriptor; tensors as for verify_attention."""
    st = load_library().mla_verify_partial(ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(page_table),
                                           _ptr(seq_lens), _ptr(tree_parent), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if st != 0:
        raise MlaError("mla_verify_partial", st)


def verify_combine(desc: MlaVerifyDesc, out, lse, workspace, stream=None) -> None:
    """Enqueue only the log-sum-exp merge (mla_verify_combine)."""
    st = load_library().mla_verify_combine(ctypes.byref(desc), _ptr(out), _ptr(lse), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if st != 0:
        raise MlaError("mla_verify_combine", st)


def build_tree_mask(tree_parent: torch.Tensor, anc_mask: torch.Tensor, dev_err: torch.Tensor | None = None,
                    stream=None) -> None:
    """Enqueue mla_build_tree_mask: anc_mask (int64 [B,T], bit patterns of the
    uint64 masks) from tree_parent (int32 [B,T])."""
    lib = load_library()
    _need(tree_parent.dtype == torch.int32 and tree_parent.is_contiguous() and tree_parent.dim() == 2,
          "tree_parent must be contiguous int32 [B,T]")
    _need(anc_mask.dtype == torch.int64 and anc_mask.is_contiguous() and anc_mask.shape == tree_parent.shape,
          "anc_mask must be contiguous int64 [B,T]")
    _need(dev_err is None or (dev_err.dtype == torch.int32 and dev_err.numel() >= 1), "dev_err must be int32")
    b, t = tree_parent.shape
    st = lib.mla_build_tree_mask(_ptr(tree_parent), _ptr(anc_mask), b, t, _ptr(dev_err), _stream_handle(stream))
    if st != 0:
        raise MlaError("mla_build_tree_mask", st)


def alloc_workspace(desc: MlaVerifyDesc, device="cuda") -> torch.Tensor:
    """A zeroed workspace of the size the descriptor needs (uint8)."""
    n = workspace_bytes(desc)
    if n == 0:
        raise ValueError("descriptor rejected by the library")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def device_error(workspace: torch.Tensor) -> int:
    """Read the sticky device error word (a device-to-host copy: call it off
    the hot path)."""
    return int(workspace[:4].view(torch.int32).item())


@dataclass
class VerifyPlan:
    """A descriptor and its workspace, made once and reused across calls (the
    capture-friendly way to call the library)."""
    desc: MlaVerifyDesc
    workspace: torch.Tensor
    page_size: int
    nsplit: int
    sm_scale: float

    @classmethod
    def create(cls, q, kv_cache, page_table, *, page_size: int, nsplit: int, sm_scale: float):
        desc = desc_for(q, kv_cache, page_table, page_size=page_size, nsplit=nsplit, sm_scale=sm_scale)
        return cls(desc, alloc_workspace(desc, q.device), page_size, nsplit, sm_scale)

    def __call__(self, q, kv_cache, page_table, seq_lens, tree_parent, out, lse, stream=None):
        verify_attention(q, kv_cache, page_table, seq_lens, tree_parent, out, lse, self.workspace,
                         page_size=self.page_size, nsplit=self.nsplit, sm_scale=self.sm_scale, stream=stream)


# ---------------------------------------------------------------- steps next to verify (mla_spec_ops.h)

def _check(name: str, st: int):
    if st != 0:
        raise MlaError(name, st)


def _i32(t: torch.Tensor, shape, what: str):
    _need(t.dtype == torch.int32 and t.is_contiguous() and tuple(t.shape) == tuple(shape) and t.is_cuda,
          f"{what} must be contiguous int32 {tuple(shape)} on the GPU")


def sparse_desc(q: torch.Tensor, kv_cache: torch.Tensor, indices: torch.Tensor, *, nsplit: int,
                sm_scale: float) -> MlaSparseDesc:
    b, h, d = q.shape
    return MlaSparseDesc(b, h, d, HEAD_DIM_V, indices.shape[1], nsplit, kv_cache.shape[0], kv_cache.stride(0),
                         sm_scale)


def alloc_sparse_workspace(desc: MlaSparseDesc, device="cuda") -> torch.Tensor:
    n = int(load_library().mla_sparse_decode_workspace_bytes(ctypes.byref(desc)))
    if n == 0:
        raise ValueError("descriptor rejected by the library")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def sparse_decode(q: torch.Tensor, kv_cache: torch.Tensor, indices: torch.Tensor, lens: torch.Tensor | None,
                  out: torch.Tensor, lse: torch.Tensor, workspace: torch.Tensor, *, nsplit: int, sm_scale: float,
                  stream=None) -> None:
    """Enqueue mla_sparse_decode: q bf16 [B,H,576], indices int32 [B,K] (-1 =
    unused), lens int32 [B] or None; writes out bf16 [B,H,512] and lse fp32 [B,H]."""
    b, h, _ = q.shape
    _need(q.dtype == torch.bfloat16 and q.is_contiguous() and q.is_cuda, "q must be contiguous bf16 [B,H,576]")
    _need(kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 2 and kv_cache.stride(1) == 1,
          "kv_cache must be bf16 [slots, stride]")
    _i32(indices, (b, indices.shape[1]), "indices")
    if lens is not None:
        _i32(lens, (b,), "lens")
    _need(out.dtype == torch.bfloat16 and out.is_contiguous() and tuple(out.shape) == (b, h, HEAD_DIM_V),
          "out must be contiguous bf16 [B,H,512]")
    _need(lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (b, h), "lse must be fp32 [B,H]")
    desc = sparse_desc(q, kv_cache, indices, nsplit=nsplit, sm_scale=sm_scale)
    _check("mla_sparse_decode", load_library().mla_sparse_decode(
        ctypes.byref(desc), _ptr(q), _ptr(kv_cache), _ptr(indices), _ptr(lens), _ptr(out), _ptr(lse),
        _ptr(workspace), workspace.numel(), _stream_handle(stream)))


def kv_append(kv_cache: torch.Tensor, new_rows: torch.Tensor, out_cache_loc: torch.Tensor,
              dev_err: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue mla_kv_append: kv_cache[out_cache_loc[r]] = new_rows[r]."""
    n = new_rows.shape[0]
    _need(kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 2 and kv_cache.stride(1) == 1,
          "kv_cache must be bf16 [slots, stride]")
    _need(new_rows.dtype == torch.bfloat16 and new_rows.is_contiguous() and new_rows.shape[1] == HEAD_DIM_QK,
          "new_rows must be contiguous bf16 [n, 576]")
    _i32(out_cache_loc, (n,), "out_cache_loc")
    _check("mla_kv_append", load_library().mla_kv_append(
        _ptr(kv_cache), kv_cache.shape[0], kv_cache.stride(0), _ptr(new_rows), _ptr(out_cache_loc), n,
        _ptr(dev_err), _stream_handle(stream)))


def tree_accept(tree_parent: torch.Tensor, draft_tokens: torch.Tensor, target_tokens: torch.Tensor,
                accept_len: torch.Tensor, accept_path: torch.Tensor, commit_tokens: torch.Tensor | None = None,
                dev_err: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue mla_tree_accept (greedy accept of each request's draft tree)."""
    b, t = tree_parent.shape
    for x, nm in ((tree_parent, "tree_parent"), (draft_tokens, "draft_tokens"), (target_tokens, "target_tokens"),
                  (accept_path, "accept_path")):
        _i32(x, (b, t), nm)
    _i32(accept_len, (b,), "accept_len")
    if commit_tokens is not None:
        _i32(commit_tokens, (b, t), "commit_tokens")
    _check("mla_tree_accept", load_library().mla_tree_accept(
        _ptr(tree_parent), _ptr(draft_tokens), _ptr(target_tokens), b, t, _ptr(accept_len), _ptr(accept_path),
        _ptr(commit_tokens), _ptr(dev_err), _stream_handle(stream)))


def commit_accepted(page_table: torch.Tensor, seq_lens: torch.Tensor, num_nodes: int, accept_len: torch.Tensor,
                    accept_path: torch.Tensor, context_lens: torch.Tensor, freed_slots: torch.Tensor | None = None,
                    kv_cache: torch.Tensor | None = None, dest_slots: torch.Tensor | None = None,
                    dev_err: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue mla_commit_accepted (page table rewritten in place; rows moved
    to dest_slots when kv_cache and dest_slots are given)."""
    b, max_pages = page_table.shape
    _i32(page_table, (b, max_pages), "page_table")
    _i32(seq_lens, (b,), "seq_lens")
    _i32(accept_len, (b,), "accept_len")
    _i32(accept_path, (b, num_nodes), "accept_path")
    _i32(context_lens, (b,), "context_lens")
    if freed_slots is not None:
        _i32(freed_slots, (b, num_nodes), "freed_slots")
    slots, stride = 0, 0
    if kv_cache is not None:
        _need(kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 2 and kv_cache.stride(1) == 1,
              "kv_cache must be bf16 [slots, stride]")
        slots, stride = kv_cache.shape[0], kv_cache.stride(0)
    if dest_slots is not None:
        _i32(dest_slots, (b, num_nodes), "dest_slots")
    _check("mla_commit_accepted", load_library().mla_commit_accepted(
        _ptr(page_table), max_pages, _ptr(seq_lens), b, num_nodes, _ptr(accept_len), _ptr(accept_path),
        _ptr(context_lens), _ptr(freed_slots), _ptr(kv_cache), slots, stride, _ptr(dest_slots), _ptr(dev_err),
        _stream_handle(stream)))


def accept_commit(tree_parent: torch.Tensor, draft_tokens: torch.Tensor, target_tokens: torch.Tensor,
                  page_table: torch.Tensor, seq_lens: torch.Tensor, accept_len: torch.Tensor,
                  accept_path: torch.Tensor, context_lens: torch.Tensor, commit_tokens: torch.Tensor | None = None,
                  freed_slots: torch.Tensor | None = None, kv_cache: torch.Tensor | None = None,
                  dest_slots: torch.Tensor | None = None, dev_err: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue mla_accept_commit: tree_accept and commit_accepted in one launch."""
    b, t = tree_parent.shape
    for x, nm in ((tree_parent, "tree_parent"), (draft_tokens, "draft_tokens"), (target_tokens, "target_tokens"),
                  (accept_path, "accept_path")):
        _i32(x, (b, t), nm)
    _need(page_table.dim() == 2 and page_table.shape[0] == b, "page_table must be [B, max_pages]")
    max_pages = page_table.shape[1]
    _i32(page_table, (b, max_pages), "page_table")
    for x, nm in ((seq_lens, "seq_lens"), (accept_len, "accept_len"), (context_lens, "context_lens")):
        _i32(x, (b,), nm)
    for x, nm in ((commit_tokens, "commit_tokens"), (freed_slots, "freed_slots"), (dest_slots, "dest_slots")):
        if x is not None:
            _i32(x, (b, t), nm)
    slots, stride = 0, 0
    if kv_cache is not None:
        _need(kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 2 and kv_cache.stride(1) == 1,
              "kv_cache must be bf16 [slots, stride]")
        slots, stride = kv_cache.shape[0], kv_cache.stride(0)
    _check("mla_accept_commit", load_library().mla_accept_commit(
        _ptr(tree_parent), _ptr(draft_tokens), _ptr(target_tokens), b, t, _ptr(page_table), max_pages,
        _ptr(seq_lens), _ptr(accept_len), _ptr(accept_path), _ptr(commit_tokens), _ptr(context_lens),
        _ptr(freed_slots), _ptr(kv_cache), slots, stride, _ptr(dest_slots), _ptr(dev_err), _stream_handle(stream)))


def window_map(target_map: torch.Tensor, lens: torch.Tensor, window: int, page: int, draft_map: torch.Tensor,
               compact_lens: torch.Tensor | None = None, dev_err: torch.Tensor | None = None, stream=None) -> None:
    """Enqueue mla_window_map: draft_map [B, window + page - 1]."""
    b, stride = target_map.shape
    _i32(target_map, (b, stride), "target_map")
    _i32(lens, (b,), "lens")
    _i32(draft_map, (b, window + page - 1), "draft_map")
    if compact_lens is not None:
        _i32(compact_lens, (b,), "compact_lens")
    _check("mla_window_map", load_library().mla_window_map(
        _ptr(target_map), stride, _ptr(lens), b, window, page, _ptr(draft_map), _ptr(compact_lens), _ptr(dev_err),
        _stream_handle(stream)))


def indexer_logits(q: torch.Tensor, weights: torch.Tensor, kv_blocks: torch.Tensor, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, logits: torch.Tensor, dev_err: torch.Tensor | None = None,
                   stream=None) -> None:
    """Enqueue mla_indexer_logits: q uint8 [B,H,128] (e4m3 codes), weights fp32
    [B,H], kv_blocks uint8 [N, 8448], block_table int32 [B, M], seq_lens int32
    [B]; writes logits fp32 [B, M*64]."""
    b, h, d = q.shape
    m = block_table.shape[1]
    _need(q.dtype == torch.uint8 and q.is_contiguous() and q.is_cuda, "q must be contiguous uint8 [B,H,128]")
    _need(weights.dtype == torch.float32 and weights.is_contiguous() and tuple(weights.shape) == (b, h),
          "weights must be fp32 [B,H]")
    _need(kv_blocks.dtype == torch.uint8 and kv_blocks.is_contiguous() and kv_blocks.dim() == 2 and
          kv_blocks.shape[1] == 8448, "kv_blocks must be contiguous uint8 [N, 8448]")
    _i32(block_table, (b, m), "block_table")
    _i32(seq_lens, (b,), "seq_lens")
    _need(logits.dtype == torch.float32 and logits.is_contiguous() and tuple(logits.shape) == (b, m * 64),
          "logits must be fp32 [B, max_blocks*64]")
    desc = MlaIndexerDesc(b, h, d, m, kv_blocks.shape[0])
    _check("mla_indexer_logits", load_library().mla_indexer_logits(
        ctypes.byref(desc), _ptr(q), _ptr(weights), _ptr(kv_blocks), _ptr(block_table), _ptr(seq_lens),
        _ptr(logits), _ptr(dev_err), _stream_handle(stream)))
