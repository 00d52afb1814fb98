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

STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_UNSUPPORTED",
          -4: "MLA_ERR_WORKSPACE", -5: "MLA_ERR_ALIGN", -6: "MLA_ERR_HIP"}


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
        lib.mla_status_string.argtypes = [ctypes.c_int]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_verify_abi_version.argtypes = []
        lib.mla_verify_abi_version.restype = i32
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
