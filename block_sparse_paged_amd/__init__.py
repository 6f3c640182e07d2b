"""Python binding of libvx, the MI355X (gfx950) block-top-k sparse paged
decode library.

Argument marshalling only: every step of the method runs in the HIP kernels
behind the C ABI declared in include/vx.h.  Tensors are passed as raw device
pointers together with the current torch stream; nothing here computes on
their contents.  The library must have been built in-tree
(``python -m block_sparse_paged_amd.build``); without it, importing the
compute entry points raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvx.so")

VX_OK = 0
VX_ERR_INVALID_ARGUMENT = 1
VX_ERR_UNSUPPORTED = 2
VX_ERR_WORKSPACE_TOO_SMALL = 3
VX_ERR_HIP = 4

VX_F32, VX_BF16 = 0, 1
VX_OP_SCORE_TOPK, VX_OP_SPARSE_DECODE, VX_OP_FULL_DECODE, VX_OP_DECODE_STEP = 0, 1, 2, 3
VX_OP_DECODE_LAYERS = 4

# Symbols include/vx.h declares (checked by the ABI tests).
EXPORTS = ("vx_centroid_update", "vx_append_kv", "vx_score_topk", "vx_score_topk_radix",
           "vx_bounds_update", "vx_score_topk_bounds",
           "vx_sparse_paged_decode",
           "vx_full_paged_decode", "vx_sparse_decode_step", "vx_sparse_decode_step_bounds",
           "vx_decode_layers", "vx_plan_decode", "vx_paged_decode_planned",
           "vx_sparse_decode_step_static",
           "vx_workspace_size", "vx_status_string", "vx_version")

# Bytes of the static device scratch behind vx_sparse_decode_step_static
# (VX_STATIC_SCRATCH_BYTES in include/vx.h).
STATIC_SCRATCH_BYTES = 32 << 20


class VxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class PagedKVStruct(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("v_aliases_k", ctypes.c_int32), ("reserved_", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("centroids", ctypes.c_void_p),
    ]


class DecodePlanStruct(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32), ("num_cus", ctypes.c_int32),
        ("pages_per_split", ctypes.c_int32), ("n_split", ctypes.c_int32),
        ("work_list", ctypes.c_int32), ("blocks", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64),
    ]


class BatchStruct(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvx.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_paged_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ, F32, VP = (ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t,
                           ctypes.c_float, ctypes.c_void_p)
    kvp, btp = P(PagedKVStruct), P(BatchStruct)
    lib.vx_centroid_update.argtypes = [kvp, VP, I32, VP]
    lib.vx_append_kv.argtypes = [kvp, btp, VP, VP, VP, VP, I32, I32, I32, VP]
    lib.vx_score_topk.argtypes = [kvp, btp, VP, I32, I32, I32, VP, VP, SZ, VP]
    lib.vx_score_topk_radix.argtypes = [kvp, btp, VP, I32, I32, I32, I32, VP, VP, VP, SZ, VP]
    lib.vx_sparse_paged_decode.argtypes = [kvp, btp, VP, VP, I32, F32, VP, VP, VP, SZ, VP]
    lib.vx_bounds_update.argtypes = [kvp, VP, VP, I32, VP]
    lib.vx_score_topk_bounds.argtypes = [kvp, btp, VP, VP, I32, I32, I32, VP, VP, SZ, VP]
    lib.vx_full_paged_decode.argtypes = [kvp, btp, VP, F32, VP, VP, VP, SZ, VP]
    lib.vx_sparse_decode_step.argtypes = [kvp, btp, VP, I32, I32, I32, I32, F32, VP, VP, VP,
                                          VP, SZ, VP]
    lib.vx_sparse_decode_step_static.argtypes = [kvp, btp, VP, I32, I32, I32, I32, F32, VP, VP,
                                                 VP, VP]
    lib.vx_sparse_decode_step_bounds.argtypes = [kvp, btp, VP, VP, I32, I32, I32, I32, F32, VP,
                                                 VP, VP, VP, SZ, VP]
    lib.vx_decode_layers.argtypes = [kvp, btp, VP, I32, VP, I32, I32, I32, I32, F32, VP, VP, VP,
                                     VP, SZ, VP]
    lib.vx_workspace_size.argtypes = [I32, kvp, btp, I32, P(SZ)]
    lib.vx_plan_decode.argtypes = [I32, kvp, btp, I32, I32, I32, P(DecodePlanStruct)]
    lib.vx_paged_decode_planned.argtypes = [kvp, btp, VP, VP, I32, P(DecodePlanStruct), F32, VP,
                                            VP, VP, SZ, VP]
    lib.vx_status_string.argtypes = [I32]
    lib.vx_status_string.restype = ctypes.c_char_p
    lib.vx_version.argtypes = []
    for name in ("vx_centroid_update", "vx_append_kv", "vx_score_topk", "vx_score_topk_radix",
                 "vx_bounds_update", "vx_score_topk_bounds",
                 "vx_sparse_paged_decode",
                 "vx_full_paged_decode", "vx_sparse_decode_step", "vx_sparse_decode_step_bounds",
                 "vx_decode_layers", "vx_plan_decode", "vx_paged_decode_planned",
                 "vx_sparse_decode_step_static", "vx_workspace_size", "vx_version"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().vx_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != VX_OK:
        raise VxError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_DT = {torch.float32: VX_F32, torch.bfloat16: VX_BF16}


@dataclass
class PagedKV:
    """The caller-owned paged KV cache and centroid table (device tensors)."""
    k_cache: torch.Tensor                  # [P, H_kv, S_p, D_qk]
    v_cache: Optional[torch.Tensor]        # [P, H_kv, S_p, D_v] or None (V = K[..., :D_v])
    centroids: torch.Tensor                # [P, H_kv, D_qk]
    head_dim_v: Optional[int] = None

    def struct(self) -> PagedKVStruct:
        k = self.k_cache
        if k.dim() != 4:
            raise ValueError(f"k_cache must be [P, H_kv, S_p, D], got shape {tuple(k.shape)}")
        if k.dtype not in _DT:
            raise ValueError(f"k_cache must be float32 or bfloat16, got {k.dtype}")
        _need(k, "k_cache")
        P, H, S, D = k.shape
        if self.v_cache is not None:
            v = self.v_cache
            _need(v, "v_cache", k.dtype)
            if v.dim() != 4 or tuple(v.shape[:3]) != (P, H, S):
                raise ValueError(f"v_cache must be [{P}, {H}, {S}, D_v], got {tuple(v.shape)}")
        if self.centroids is not None:
            _need(self.centroids, "centroids", k.dtype)
            if tuple(self.centroids.shape) != (P, H, D):
                raise ValueError(f"centroids must be [{P}, {H}, {D}], got "
                                 f"{tuple(self.centroids.shape)}")
        dv = self.v_cache.shape[-1] if self.v_cache is not None else (self.head_dim_v or D)
        return PagedKVStruct(
            dtype=_DT[k.dtype], num_pages=P, page_size=S, num_kv_heads=H,
            head_dim_qk=D, head_dim_v=dv, v_aliases_k=1 if self.v_cache is None else 0,
            reserved_=0, k_cache=k.data_ptr(),
            v_cache=None if self.v_cache is None else self.v_cache.data_ptr(),
            centroids=None if self.centroids is None else self.centroids.data_ptr())


@dataclass
class Batch:
    """Decode-batch metadata: page table and sequence lengths (device int32)."""
    page_table: torch.Tensor               # [B, max_pages] int32
    seq_lens: torch.Tensor                 # [B] int32
    num_q_heads: int
    max_seq_len: int                       # host-side bound used for planning

    def struct(self) -> BatchStruct:
        if self.page_table.dim() != 2:
            raise ValueError("page_table must be [B, max_pages]")
        _need(self.page_table, "page_table", torch.int32)
        _need(self.seq_lens, "seq_lens", torch.int32)
        B, mp = self.page_table.shape
        if tuple(self.seq_lens.shape) != (B,):
            raise ValueError(f"seq_lens must be [{B}], got {tuple(self.seq_lens.shape)}")
        return BatchStruct(batch=B, num_q_heads=self.num_q_heads, max_pages_per_req=mp,
                           max_seq_len=int(self.max_seq_len),
                           page_table=self.page_table.data_ptr(),
                           seq_lens=self.seq_lens.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _args(kv: "PagedKV", batch: "Batch", q=None, out=None, sel=None, lse=None):
    """Checks the tensors of a call against the cache and batch shapes: q
    [B, H_q, D_qk] and out [B, H_q, D_v] in the cache dtype, sel int32
    [B, H_kv, k_tot], lse float32 [B, H_q]; every tensor contiguous."""
    k = kv.k_cache
    B = batch.page_table.shape[0]
    H_q, H_kv, D = batch.num_q_heads, k.shape[1], k.shape[3]
    Dv = kv.v_cache.shape[-1] if kv.v_cache is not None else (kv.head_dim_v or D)
    if q is not None:
        _need(q, "q", k.dtype, (B, H_q, D))
    if out is not None:
        _need(out, "out", k.dtype, (B, H_q, Dv))
    if sel is not None:
        _need(sel, "sel", torch.int32)
        if sel.dim() != 3 or tuple(sel.shape[:2]) != (B, H_kv):
            raise ValueError(f"sel must be [{B}, {H_kv}, k_tot], got {tuple(sel.shape)}")
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H_q))


def workspace_size(op: int, kv: PagedKV, batch: Batch, k_tot: int = 0) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    kvs, bs = kv.struct(), batch.struct()
    _check(lib.vx_workspace_size(op, ctypes.byref(kvs), ctypes.byref(bs), k_tot,
                                 ctypes.byref(out)), "vx_workspace_size")
    return int(out.value)


def alloc_workspace(op: int, kv: PagedKV, batch: Batch, k_tot: int = 0) -> torch.Tensor:
    n = workspace_size(op, kv, batch, k_tot)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=kv.k_cache.device)


def centroid_update(kv: PagedKV, page_ids: torch.Tensor, stream=None):
    """vx_centroid_update: centroids of the listed (full) physical pages."""
    prepare_centroid_update(kv, page_ids, stream)()


def append_kv(kv: PagedKV, batch: Batch, k_src: torch.Tensor, v_src: Optional[torch.Tensor],
              src_start: torch.Tensor, n_new: torch.Tensor, max_new: int,
              update_centroids: bool = True, stream=None):
    """vx_append_kv: request b's last n_new[b] tokens (lengths from batch,
    after the write) from rows src_start[b].. of k_src / v_src into the
    cache, with the centroids of the pages the write fills."""
    prepare_append_kv(kv, batch, k_src, v_src, src_start, n_new, max_new, update_centroids,
                      stream)()


def prepare_append_kv(kv: PagedKV, batch: Batch, k_src, v_src, src_start, n_new, max_new,
                      update_centroids=True, stream=None) -> "PreparedCall":
    _need(k_src, "k_src")
    if v_src is not None:
        _need(v_src, "v_src")
    _need(src_start, "src_start", torch.int32)
    _need(n_new, "n_new", torch.int32)
    kvs, bs = kv.struct(), batch.struct()
    lib = load_library()
    args = (ctypes.byref(kvs), ctypes.byref(bs), _ptr(k_src), _ptr(v_src), _ptr(src_start),
            _ptr(n_new), k_src.shape[0], int(max_new), int(bool(update_centroids)),
            _stream(stream))
    return PreparedCall(lib.vx_append_kv, args, "vx_append_kv",
                        (kvs, bs, kv, batch, k_src, v_src, src_start, n_new))


def score_topk(kv: PagedKV, batch: Batch, q: torch.Tensor, topk: int, n_bos: int,
               n_eos: int, sel: torch.Tensor, workspace: torch.Tensor, stream=None):
    """vx_score_topk: selected logical pages per (request, KV head) into sel."""
    prepare_score_topk(kv, batch, q, topk, n_bos, n_eos, sel, workspace, stream)()


def score_topk_radix(kv: PagedKV, batch: Batch, q: torch.Tensor, topk: int, n_bos: int,
                     n_eos: int, levels: int, rnd: torch.Tensor, sel: torch.Tensor,
                     workspace: torch.Tensor, stream=None):
    """vx_score_topk_radix: the lossy radix top-k (``levels`` histogram
    levels, then the boundary bin's members by rank from ``rnd``) into sel.
    ``rnd`` holds one random 32-bit word per (request, KV head) (int32 or
    uint32 tensor of B * H_kv elements, read as uint32)."""
    prepare_score_topk_radix(kv, batch, q, topk, n_bos, n_eos, levels, rnd, sel, workspace,
                             stream)()


def bounds_update(kv: PagedKV, bounds: torch.Tensor, page_ids: torch.Tensor, stream=None):
    """vx_bounds_update: per-channel key minimum and maximum of the listed
    (full) physical pages into ``bounds`` [P, H_kv, 2, D] (Quest's summary)."""
    _need(bounds, "bounds", kv.k_cache.dtype)
    _need(page_ids, "page_ids", torch.int32)
    kvs = kv.struct()
    _check(load_library().vx_bounds_update(ctypes.byref(kvs), _ptr(bounds), _ptr(page_ids),
                                           page_ids.numel(), _stream(stream)),
           "vx_bounds_update")


def prepare_score_topk_bounds(kv: PagedKV, batch: Batch, bounds, q, topk, n_bos, n_eos, sel,
                              workspace, stream=None) -> "PreparedCall":
    _args(kv, batch, q=q, sel=sel)
    _need(bounds, "bounds", kv.k_cache.dtype)
    kvs, bs = kv.struct(), batch.struct()
    lib = load_library()
    args = (ctypes.byref(kvs), ctypes.byref(bs), _ptr(bounds), _ptr(q), topk, n_bos, n_eos,
            _ptr(sel), _ptr(workspace), workspace.numel(), _stream(stream))
    return PreparedCall(lib.vx_score_topk_bounds, args, "vx_score_topk_bounds",
                        (kvs, bs, kv, batch, bounds, q, sel, workspace))


def score_topk_bounds(kv: PagedKV, batch: Batch, bounds: torch.Tensor, q: torch.Tensor,
                      topk: int, n_bos: int, n_eos: int, sel: torch.Tensor,
                      workspace: torch.Tensor, stream=None):
    """vx_score_topk_bounds: pages selected by Quest's criticality bound."""
    prepare_score_topk_bounds(kv, batch, bounds, q, topk, n_bos, n_eos, sel, workspace, stream)()


def sparse_paged_decode(kv: PagedKV, batch: Batch, q: torch.Tensor, sel: torch.Tensor,
                        sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor],
                        workspace: torch.Tensor, stream=None):
    """vx_sparse_paged_decode: attention over the pages listed in sel."""
    prepare_sparse_paged_decode(kv, batch, q, sel, sm_scale, out, lse, workspace, stream)()


def full_paged_decode(kv: PagedKV, batch: Batch, q: torch.Tensor, sm_scale: float,
                      out: torch.Tensor, lse: Optional[torch.Tensor],
                      workspace: torch.Tensor, stream=None):
    """vx_full_paged_decode: attention over every page (the dense baseline)."""
    prepare_full_paged_decode(kv, batch, q, sm_scale, out, lse, workspace, stream)()


def sparse_decode_step(kv: PagedKV, batch: Batch, q: torch.Tensor, topk: int, n_bos: int,
                       n_eos: int, update_completed: bool, sm_scale: float, sel: torch.Tensor,
                       out: torch.Tensor, lse: Optional[torch.Tensor], workspace: torch.Tensor,
                       stream=None):
    """vx_sparse_decode_step: completed-page centroids, selection and attention."""
    prepare_sparse_decode_step(kv, batch, q, topk, n_bos, n_eos, update_completed, sm_scale,
                               sel, out, lse, workspace, stream)()


def sparse_decode_step_static(kv: PagedKV, batch: Batch, q: torch.Tensor, topk: int, n_bos: int,
                              n_eos: int, update_completed: bool, sm_scale: float,
                              sel: torch.Tensor, out: torch.Tensor, lse: Optional[torch.Tensor],
                              stream=None):
    """vx_sparse_decode_step_static: the decode step with the library's static
    device scratch as its workspace (no allocation; calls that overlap on one
    GPU race)."""
    _args(kv, batch, q=q, sel=sel, out=out, lse=lse)
    kvs, bs = kv.struct(), batch.struct()
    _check(load_library().vx_sparse_decode_step_static(
        ctypes.byref(kvs), ctypes.byref(bs), _ptr(q), topk, n_bos, n_eos,
        1 if update_completed else 0, float(sm_scale), _ptr(sel), _ptr(out), _ptr(lse),
        _stream(stream)), "vx_sparse_decode_step_static")


def sparse_decode_step_bounds(kv: PagedKV, batch: Batch, bounds: torch.Tensor, q: torch.Tensor,
                              topk: int, n_bos: int, n_eos: int, update_completed: bool,
                              sm_scale: float, sel: torch.Tensor, out: torch.Tensor,
                              lse: Optional[torch.Tensor], workspace: torch.Tensor, stream=None):
    """vx_sparse_decode_step_bounds: the decode step under Quest's key-bounds
    rule (completed pages' bounds, selection and attention)."""
    prepare_sparse_decode_step_bounds(kv, batch, bounds, q, topk, n_bos, n_eos, update_completed,
                                      sm_scale, sel, out, lse, workspace, stream)()


def plan_decode(op: int, kv: PagedKV, batch: Batch, k_tot: int = 0, num_cus: int = 0,
                pages_per_split: int = 0) -> DecodePlanStruct:
    """vx_plan_decode: the launch plan of a sparse (VX_OP_SPARSE_DECODE) or
    dense (VX_OP_FULL_DECODE) decode call on a GPU of ``num_cus`` compute
    units (0: the current device), optionally with a fixed split size."""
    plan = DecodePlanStruct()
    kvs, bs = kv.struct(), batch.struct()
    _check(load_library().vx_plan_decode(op, ctypes.byref(kvs), ctypes.byref(bs), int(k_tot),
                                         int(num_cus), int(pages_per_split), ctypes.byref(plan)),
           "vx_plan_decode")
    return plan


def paged_decode_planned(kv: PagedKV, batch: Batch, q: torch.Tensor, sel: Optional[torch.Tensor],
                         plan: DecodePlanStruct, sm_scale: float, out: torch.Tensor,
                         lse: Optional[torch.Tensor], workspace: torch.Tensor, stream=None):
    """vx_paged_decode_planned: the sparse (sel given) or dense (sel None)
    decode with an explicit plan from plan_decode."""
    _args(kv, batch, q=q, out=out, sel=sel, lse=lse)
    kvs, bs = kv.struct(), batch.struct()
    _check(load_library().vx_paged_decode_planned(
        ctypes.byref(kvs), ctypes.byref(bs), _ptr(q), _ptr(sel),
        0 if sel is None else sel.shape[-1], ctypes.byref(plan), float(sm_scale), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)), "vx_paged_decode_planned")


def version() -> int:
    return int(load_library().vx_version())


class PreparedCall:
    """A libvx call with its arguments marshalled once; calling it only
    crosses the C ABI.  Holds references to every struct and tensor it
    points at."""

    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, fn, args, name, keep):
        self._fn, self._args, self._name, self._keep = fn, args, name, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != VX_OK:
            raise VxError(st, self._name)


def prepare_centroid_update(kv: PagedKV, page_ids: torch.Tensor, stream=None) -> PreparedCall:
    _need(page_ids, "page_ids", torch.int32)
    kvs = kv.struct()
    lib = load_library()
    args = (ctypes.byref(kvs), _ptr(page_ids), page_ids.numel(), _stream(stream))
    return PreparedCall(lib.vx_centroid_update, args, "vx_centroid_update", (kvs, kv, page_ids))


def prepare_score_topk(kv: PagedKV, batch: Batch, q, topk, n_bos, n_eos, sel, workspace,
                       stream=None) -> PreparedCall:
    _args(kv, batch, q=q, sel=sel)
    kvs, bs = kv.struct(), batch.struct()
    lib = load_library()
    args = (ctypes.byref(kvs), ctypes.byref(bs), _ptr(q), topk, n_bos, n_eos, _ptr(sel),
            _ptr(workspace), workspace.numel(), _stream(stream))
    return PreparedCall(lib.vx_score_topk, args, "vx_score_topk",
                        (kvs, bs, kv, batch, q, sel, workspace))


def prepare_score_topk_radix(kv: PagedKV, batch: Batch, q, topk, n_bos, n_eos, levels, rnd,
                             sel, workspace, stream=None) -> PreparedCall:
    _args(kv, batch, q=q, sel=sel)
    if rnd.device.type != "cuda" or not rnd.is_contiguous() or rnd.element_size() != 4 or \
            rnd.dtype.is_floating_point:
        raise ValueError("rnd must be a contiguous 32-bit integer CUDA tensor")
    kvs, bs = kv.struct(), batch.struct()
    if rnd.numel() < bs.batch * kvs.num_kv_heads:
        raise ValueError("rnd needs one word per (request, KV head)")
    lib = load_library()
    args = (ctypes.byref(kvs), ctypes.byref(bs), _ptr(q), topk, n_bos, n_eos, levels, _ptr(rnd),
            _ptr(sel), _ptr(workspace), workspace.numel(), _stream(stream))
    return PreparedCall(lib.vx_score_topk_radix, args, "vx_score_topk_radix",
                        (kvs, bs, kv, batch, q, rnd, sel, workspace))


def prepare_sparse_paged_decode(kv: PagedKV, batch: Batch, q, sel, sm_scale, out, lse,
                                workspace, stream=None) -> PreparedCall:
    _args(kv, batch, q=q, sel=sel, out=out, lse=lse)
    kvs, bs = kv.struct(), batch.struct()
    lib = load_library()
    args = (ctypes.byref(kvs), ctypes.byref(bs), _ptr(q), _ptr(sel), sel.shape[-1],
            float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
            _stream(stream))
    return PreparedCall(lib.vx_sparse_paged_decode, args, "vx_sparse_paged_decode",
                        (kvs, bs, kv, batch, q, sel, out, lse, workspace))


def prepare_full_paged_decode(kv: PagedKV, batch: Batch, q, sm_scale, out, lse, workspace,
                              stream=None) -> PreparedCall:
    _args(kv, batch, q=q, out=out, lse=lse)
    kvs, bs = kv.struct(), batch.struct()
    lib = load_library()
    args = (ctypes.byref(kvs), ctypes.byref(bs), _ptr(q), float(sm_scale), _ptr(out),
            _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream))
    return PreparedCall(lib.vx_full_paged_decode, args, "vx_full_paged_decode",
                        (kvs, bs, kv, batch, q, out, lse, workspace))


def prepare_sparse_decode_step(kv: PagedKV, batch: Batch, q, topk, n_bos, n_eos,
                               update_completed, sm_scale, sel, out, lse, workspace,
                               stream=None) -> PreparedCall:
    _args(kv, batch, q=q, sel=sel, out=out, lse=lse)
    kvs, bs = kv.struct(), batch.struct()
    lib = load_library()
    args = (ctypes.byref(kvs), ctypes.byref(bs), _ptr(q), topk, n_bos, n_eos,
            1 if update_completed else 0, float(sm_scale), _ptr(sel), _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream(stream))
    return PreparedCall(lib.vx_sparse_decode_step, args, "vx_sparse_decode_step",
                        (kvs, bs, kv, batch, q, sel, out, lse, workspace))


def prepare_sparse_decode_step_bounds(kv: PagedKV, batch: Batch, bounds, q, topk, n_bos, n_eos,
                                      update_completed, sm_scale, sel, out, lse, workspace,
                                      stream=None) -> PreparedCall:
    _args(kv, batch, q=q, sel=sel, out=out, lse=lse)
    _need(bounds, "bounds", kv.k_cache.dtype)
    kvs, bs = kv.struct(), batch.struct()
    lib = load_library()
    args = (ctypes.byref(kvs), ctypes.byref(bs), _ptr(bounds), _ptr(q), topk, n_bos, n_eos,
            1 if update_completed else 0, float(sm_scale), _ptr(sel), _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream(stream))
    return PreparedCall(lib.vx_sparse_decode_step_bounds, args, "vx_sparse_decode_step_bounds",
                        (kvs, bs, kv, batch, bounds, q, sel, out, lse, workspace))


def prepare_decode_layers(kvs: list, batch: Batch, qs: list, dense: Optional[list], topk: int,
                          n_bos: int, n_eos: int, update_completed: bool, sm_scale: float,
                          sels: Optional[list], outs: list, lses: Optional[list],
                          workspace: torch.Tensor, stream=None) -> PreparedCall:
    """vx_decode_layers over len(kvs) layers: layer l runs full attention
    when dense[l] is true, else the fused sparse step into sels[l].  The
    host arrays of structs and pointers are built here, once."""
    n = len(kvs)
    if len(qs) != n or len(outs) != n or (dense is not None and len(dense) != n) or \
            (sels is not None and len(sels) != n) or (lses is not None and len(lses) != n):
        raise ValueError("one entry per layer in every list")
    for t in list(qs) + list(outs):
        _need(t, "q/out")
    for t in (sels or []):
        if t is not None:
            _need(t, "sel", torch.int32)
    kv_arr = (PagedKVStruct * max(n, 1))(*[kv.struct() for kv in kvs])
    bs = batch.struct()
    VPA = ctypes.c_void_p * max(n, 1)
    q_arr = VPA(*[t.data_ptr() for t in qs])
    out_arr = VPA(*[t.data_ptr() for t in outs])
    sel_arr = None if sels is None else VPA(*[0 if t is None else t.data_ptr() for t in sels])
    lse_arr = None if lses is None else VPA(*[0 if t is None else t.data_ptr() for t in lses])
    dense_arr = None if dense is None else (ctypes.c_uint8 * max(n, 1))(*[1 if d else 0 for d in dense])
    lib = load_library()
    args = (kv_arr, ctypes.byref(bs), q_arr, n, dense_arr, topk, n_bos, n_eos,
            1 if update_completed else 0, float(sm_scale), sel_arr, out_arr, lse_arr,
            _ptr(workspace), workspace.numel(), _stream(stream))
    return PreparedCall(lib.vx_decode_layers, args, "vx_decode_layers",
                        (kv_arr, bs, q_arr, out_arr, sel_arr, lse_arr, dense_arr, list(kvs), batch,
                         list(qs), list(outs), list(sels or []), list(lses or []), workspace))


def decode_layers(kvs: list, batch: Batch, qs: list, dense: Optional[list], topk: int,
                  n_bos: int, n_eos: int, update_completed: bool, sm_scale: float,
                  sels: Optional[list], outs: list, lses: Optional[list],
                  workspace: torch.Tensor, stream=None):
    """vx_decode_layers: one decode step through several attention layers."""
    prepare_decode_layers(kvs, batch, qs, dense, topk, n_bos, n_eos, update_completed, sm_scale,
                          sels, outs, lses, workspace, stream)()


def capture_graph(make_call) -> "torch.cuda.CUDAGraph":
    """Capture the libvx launches of ``make_call(stream)()`` into a graph.

    ``make_call`` receives the capturing stream and returns a prepared call
    (for instance ``lambda s: prepare_decode_layers(..., stream=s)``); the
    call is made once on a side stream first, so that every one-time host
    query happens outside the capture.  Replaying the graph repeats the
    launches with the pointers, lengths bound and plan of the capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        make_call(side)()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        make_call(torch.cuda.current_stream())()
    return g
