"""ctypes binding of libkvs (include/kvs.h), argument marshalling only.

Every function has the name and argument order of its C entry point; torch
tensors are accepted where the C call takes a pointer and are checked for
device, dtype, size and contiguity before their data pointers are passed.
Nothing here computes any part of the method: the work runs in the HIP
kernels of libkvs.so, and importing this module fails loudly when that
library has not been built.

torch is imported before the library is opened so that libkvs.so binds to
the HIP runtime torch already loaded (one runtime per process).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvs.so")

KVS_OK, KVS_ERR_INVALID_ARG, KVS_ERR_UNSUPPORTED, KVS_ERR_CAPACITY, KVS_ERR_HIP = range(5)
KVS_F32, KVS_BF16, KVS_FP8_E4M3 = 0, 1, 2
KVS_TABLE_PAGED, KVS_TABLE_HOT = 0, 1
KVS_DEVERR_SEQLEN, KVS_DEVERR_TABLE, KVS_DEVERR_SEL = 0x1, 0x2, 0x4

DTYPE_CODE = {"f32": KVS_F32, "bf16": KVS_BF16, "e4m3": KVS_FP8_E4M3}
_TORCH_OF = {KVS_F32: torch.float32, KVS_BF16: torch.bfloat16, KVS_FP8_E4M3: torch.uint8}


class KvsError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: {detail} (status {status})")
        self.status = status


class _CLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "max_blocks",
        "num_pages", "q_dtype", "kv_dtype", "quant_group")]


@dataclass(frozen=True)
class Layout:
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    max_blocks: int
    num_pages: int
    q_dtype: int
    kv_dtype: int
    quant_group: int = 0

    def c(self) -> _CLayout:
        return _CLayout(self.num_seqs, self.num_q_heads, self.num_kv_heads, self.head_dim,
                        self.block_size, self.max_blocks, self.num_pages, self.q_dtype,
                        self.kv_dtype, self.quant_group)

    @property
    def summary_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.kv_dtype == KVS_BF16 else torch.float32

    def summary_dtype_of(self, kind: int) -> torch.dtype:
        return torch.float32 if kind == KVS_SUMM_MEAN else self.summary_dtype

    def summary_numel(self, kind: int = 0) -> int:
        """Elements of the summary table: [B][Hkv][MB][2][D] (min/max) or
        [B][Hkv][MB][D] (mean)."""
        n = self.num_seqs * self.num_kv_heads * self.max_blocks * self.head_dim
        return n if kind == KVS_SUMM_MEAN else 2 * n


class _CAppendArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_new", "v_new", "k_new_scales", "v_new_scales", "block_table", "k_pool", "v_pool",
        "k_scales", "v_scales", "host_k", "host_v", "host_k_scales", "host_v_scales")]


class _CHotLive(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_pool", "v_pool", "k_scales", "v_scales", "block_table", "seq_lens")]


class _CSelectOpts(ctypes.Structure):
    _fields_ = [("recent_blocks", ctypes.c_int32), ("use_ema", ctypes.c_int32),
                ("ema_alpha", ctypes.c_double), ("ema_state", ctypes.c_void_p),
                ("summary_kind", ctypes.c_int32), ("accumulate", ctypes.c_int32)]


KVS_SUMM_MINMAX, KVS_SUMM_MEAN = 0, 1


@dataclass
class AppendArgs:
    """Tensors of kvs_append_args (include/kvs.h); host_* are pinned host
    tensors or None (no sealing)."""
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_new_scales: torch.Tensor | None
    v_new_scales: torch.Tensor | None
    block_table: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_scales: torch.Tensor | None = None
    v_scales: torch.Tensor | None = None
    host_k: torch.Tensor | None = None
    host_v: torch.Tensor | None = None
    host_k_scales: torch.Tensor | None = None
    host_v_scales: torch.Tensor | None = None


@dataclass
class HotLive:
    """Tensors of kvs_hot_live (include/kvs.h): the paged device cache the
    hot-buffer swap-in copies each sequence's newest block from."""
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_scales: torch.Tensor | None
    v_scales: torch.Tensor | None
    block_table: torch.Tensor
    seq_lens: torch.Tensor


@dataclass
class SelectOpts:
    """kvs_select_opts: recent window, score smoothing, summary kind,
    cross-layer accumulation (kvs_score_blocks)."""
    recent_blocks: int = 1
    use_ema: bool = False
    ema_alpha: float = 0.7
    ema_state: torch.Tensor | None = None
    summary_kind: int = 0  # KVS_SUMM_MINMAX or KVS_SUMM_MEAN
    accumulate: bool = False


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python -m query_aware_sparse_kvs_amd.build)")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_LOCAL)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    LP = ctypes.POINTER(_CLayout)
    sigs = {
        "kvs_build_summaries": (i32, [LP, P, P, P, P, P, i32, P, P]),
        "kvs_build_summaries_ex": (i32, [LP, i32, P, P, P, P, P, i32, P, P]),
        "kvs_select_topk": (i32, [LP, P, P, P, i32, P, P, P, sz, P]),
        "kvs_select_topk_append": (i32, [LP, P, P, P, P, P, P, i32, P, P, P, sz, P]),
        "kvs_sparse_decode_attn": (i32, [LP, i32, P, P, P, P, P, P, P, P, i32, ctypes.c_float, P, P, sz, P]),
        "kvs_sparse_decode_attn_noalloc": (i32, [LP, i32, P, P, P, P, P, P, P, P, i32, ctypes.c_float, P, P]),
        "kvs_append_token": (i32, [LP, ctypes.POINTER(_CAppendArgs), P, P, P]),
        "kvs_append_sparse_decode_attn": (i32, [LP, ctypes.POINTER(_CAppendArgs), P, P, P, P, i32, ctypes.c_float,
                                                P, P, sz, P]),
        "kvs_score_blocks": (i32, [LP, P, P, P, ctypes.POINTER(_CSelectOpts), ctypes.POINTER(_CAppendArgs),
                                   P, P, P]),
        "kvs_select_attn": (i32, [LP, P, P, P, P, P, P, P, P, i32, i32, P, ctypes.c_float, P, P, sz, P]),
        "kvs_select_topk_ex": (i32, [LP, P, P, P, i32, ctypes.POINTER(_CSelectOpts),
                                     ctypes.POINTER(_CAppendArgs), P, P, P, sz, P]),
        "kvs_hot_lookup_swapin": (i32, [LP, P, i32, i32, i64, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]),
        "kvs_hot_lookup": (i32, [LP, P, i32, i32, i64, P, P, P, P, P, P]),
        "kvs_hot_swapin": (i32, [LP, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, P]),
        "kvs_select_workspace_size": (sz, [LP, i32]),
        "kvs_attn_workspace_size": (sz, [LP, i32]),
        "kvs_attn_num_splits": (i32, [LP, i32]),
        "kvs_select_uses_matrix_cores": (i32, [LP, i32]),
        "kvs_device_errors": (i32, [ctypes.POINTER(ctypes.c_uint32), i32, P]),
        "kvs_status_string": (ctypes.c_char_p, [i32]),
        "kvs_last_error": (ctypes.c_char_p, []),
        "kvs_abi_version": (i32, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()
EXPORTED = ("kvs_build_summaries", "kvs_select_topk", "kvs_select_topk_append", "kvs_sparse_decode_attn",
            "kvs_sparse_decode_attn_noalloc", "kvs_hot_lookup_swapin", "kvs_hot_lookup", "kvs_hot_swapin",
            "kvs_append_token", "kvs_append_sparse_decode_attn", "kvs_select_topk_ex", "kvs_score_blocks",
            "kvs_select_attn",
            "kvs_build_summaries_ex", "kvs_select_uses_matrix_cores",
            "kvs_select_workspace_size", "kvs_attn_workspace_size", "kvs_attn_num_splits",
            "kvs_device_errors", "kvs_status_string", "kvs_last_error", "kvs_abi_version")


def library():
    return _lib


def _check(status: int, what: str) -> None:
    if status != KVS_OK:
        raise KvsError(status, what, _lib.kvs_last_error().decode())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, name, dtype=None, numel=None, device=True, pinned=False):
    """Data pointer of a contiguous tensor after the checks; None for None."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or None")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not device and t.is_cuda:
        raise ValueError(f"{name} must be a host tensor")
    if pinned and not t.is_pinned():
        raise ValueError(f"{name} must be pinned host memory")
    return ctypes.c_void_p(t.data_ptr())


def _pool_dtype(L: Layout):
    return _TORCH_OF[L.kv_dtype]


def kvs_build_summaries(layout: Layout, k_pool, k_scales, block_table, seq_lens, first_block,
                        num_rebuild: int, summaries, stream=None) -> None:
    L = layout
    tile = L.num_kv_heads * L.block_size * L.head_dim
    qg = L.quant_group
    _check(_lib.kvs_build_summaries(
        ctypes.byref(L.c()),
        _ptr(k_pool, "k_pool", _pool_dtype(L), L.num_pages * tile),
        _ptr(k_scales, "k_scales", torch.float32, L.num_pages * tile // qg if qg else None),
        _ptr(block_table, "block_table", torch.int32, L.num_seqs * L.max_blocks),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        _ptr(first_block, "first_block", torch.int32, L.num_seqs),
        int(num_rebuild),
        _ptr(summaries, "summaries", L.summary_dtype, L.num_seqs * L.num_kv_heads * L.max_blocks * 2 * L.head_dim),
        _stream(stream)), "kvs_build_summaries")


def kvs_build_summaries_ex(layout: Layout, summary_kind: int, k_pool, k_scales, block_table, seq_lens,
                           first_block, num_rebuild: int, summaries, stream=None) -> None:
    L = layout
    tile = L.num_kv_heads * L.block_size * L.head_dim
    qg = L.quant_group
    _check(_lib.kvs_build_summaries_ex(
        ctypes.byref(L.c()), int(summary_kind),
        _ptr(k_pool, "k_pool", _pool_dtype(L), L.num_pages * tile),
        _ptr(k_scales, "k_scales", torch.float32, L.num_pages * tile // qg if qg else None),
        _ptr(block_table, "block_table", torch.int32, L.num_seqs * L.max_blocks),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        _ptr(first_block, "first_block", torch.int32, L.num_seqs),
        int(num_rebuild),
        _ptr(summaries, "summaries", L.summary_dtype_of(summary_kind), L.summary_numel(summary_kind)),
        _stream(stream)), "kvs_build_summaries_ex")


def kvs_select_topk(layout: Layout, q, summaries, seq_lens, k: int, sel, bounds_out, workspace,
                    stream=None) -> None:
    L = layout
    ws = _ptr(workspace, "workspace", torch.uint8)
    _check(_lib.kvs_select_topk(
        ctypes.byref(L.c()),
        _ptr(q, "q", _TORCH_OF[L.q_dtype], L.num_seqs * L.num_q_heads * L.head_dim),
        _ptr(summaries, "summaries", L.summary_dtype, L.num_seqs * L.num_kv_heads * L.max_blocks * 2 * L.head_dim),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        int(k),
        _ptr(sel, "sel", torch.int32, L.num_seqs * L.num_kv_heads * k),
        _ptr(bounds_out, "bounds_out", torch.float64, L.num_seqs * L.num_kv_heads * L.max_blocks),
        ws, workspace.numel() if workspace is not None else 0,
        _stream(stream)), "kvs_select_topk")


def kvs_select_topk_append(layout: Layout, q, k_pool, k_scales, block_table, seq_lens, summaries, k: int,
                           sel, bounds_out, workspace, stream=None) -> None:
    L = layout
    tile = L.num_kv_heads * L.block_size * L.head_dim
    qg = L.quant_group
    ws = _ptr(workspace, "workspace", torch.uint8)
    _check(_lib.kvs_select_topk_append(
        ctypes.byref(L.c()),
        _ptr(q, "q", _TORCH_OF[L.q_dtype], L.num_seqs * L.num_q_heads * L.head_dim),
        _ptr(k_pool, "k_pool", _pool_dtype(L), L.num_pages * tile),
        _ptr(k_scales, "k_scales", torch.float32, L.num_pages * tile // qg if qg else None),
        _ptr(block_table, "block_table", torch.int32, L.num_seqs * L.max_blocks),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        _ptr(summaries, "summaries", L.summary_dtype, L.num_seqs * L.num_kv_heads * L.max_blocks * 2 * L.head_dim),
        int(k),
        _ptr(sel, "sel", torch.int32, L.num_seqs * L.num_kv_heads * k),
        _ptr(bounds_out, "bounds_out", torch.float64, L.num_seqs * L.num_kv_heads * L.max_blocks),
        ws, workspace.numel() if workspace is not None else 0,
        _stream(stream)), "kvs_select_topk_append")


def _live_struct(L: Layout, a: HotLive | None):
    if a is None:
        return None
    tile = L.num_kv_heads * L.block_size * L.head_dim
    qg = L.quant_group
    dt = _pool_dtype(L)
    return ctypes.byref(_CHotLive(
        _ptr(a.k_pool, "live k_pool", dt, L.num_pages * tile),
        _ptr(a.v_pool, "live v_pool", dt, L.num_pages * tile),
        _ptr(a.k_scales, "live k_scales", torch.float32, L.num_pages * tile // qg if qg else None),
        _ptr(a.v_scales, "live v_scales", torch.float32, L.num_pages * tile // qg if qg else None),
        _ptr(a.block_table, "live block_table", torch.int32, L.num_seqs * L.max_blocks),
        _ptr(a.seq_lens, "live seq_lens", torch.int32, L.num_seqs)))


def _append_struct(L: Layout, a: AppendArgs) -> _CAppendArgs:
    units = L.num_seqs * L.num_kv_heads
    tile = L.num_kv_heads * L.block_size * L.head_dim
    qg = L.quant_group
    host_n = units * L.max_blocks * L.block_size * L.head_dim
    dt = _pool_dtype(L)
    return _CAppendArgs(
        _ptr(a.k_new, "k_new", dt, units * L.head_dim),
        _ptr(a.v_new, "v_new", dt, units * L.head_dim),
        _ptr(a.k_new_scales, "k_new_scales", torch.float32, units * L.head_dim // qg if qg else None),
        _ptr(a.v_new_scales, "v_new_scales", torch.float32, units * L.head_dim // qg if qg else None),
        _ptr(a.block_table, "block_table", torch.int32, L.num_seqs * L.max_blocks),
        _ptr(a.k_pool, "k_pool", dt, L.num_pages * tile),
        _ptr(a.v_pool, "v_pool", dt, L.num_pages * tile),
        _ptr(a.k_scales, "k_scales", torch.float32, L.num_pages * tile // qg if qg else None),
        _ptr(a.v_scales, "v_scales", torch.float32, L.num_pages * tile // qg if qg else None),
        _ptr(a.host_k, "host_k", dt, host_n, device=False, pinned=True),
        _ptr(a.host_v, "host_v", dt, host_n, device=False, pinned=True),
        _ptr(a.host_k_scales, "host_k_scales", torch.float32, host_n // qg if qg else None, device=False,
             pinned=True),
        _ptr(a.host_v_scales, "host_v_scales", torch.float32, host_n // qg if qg else None, device=False,
             pinned=True))


def kvs_append_token(layout: Layout, append: AppendArgs, seq_lens, summaries, stream=None) -> None:
    L = layout
    ca = _append_struct(L, append)
    _check(_lib.kvs_append_token(
        ctypes.byref(L.c()), ctypes.byref(ca),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        _ptr(summaries, "summaries", L.summary_dtype, L.num_seqs * L.num_kv_heads * L.max_blocks * 2 * L.head_dim),
        _stream(stream)), "kvs_append_token")


def kvs_append_sparse_decode_attn(layout: Layout, append: AppendArgs, summaries, q, seq_lens, sel, k: int,
                                  sm_scale: float, out, workspace, stream=None) -> None:
    L = layout
    ca = _append_struct(L, append)
    _check(_lib.kvs_append_sparse_decode_attn(
        ctypes.byref(L.c()), ctypes.byref(ca),
        _ptr(summaries, "summaries", L.summary_dtype, L.num_seqs * L.num_kv_heads * L.max_blocks * 2 * L.head_dim),
        _ptr(q, "q", _TORCH_OF[L.q_dtype], L.num_seqs * L.num_q_heads * L.head_dim),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        _ptr(sel, "sel", torch.int32, L.num_seqs * L.num_kv_heads * k),
        k, float(sm_scale),
        _ptr(out, "out", torch.float32, L.num_seqs * L.num_q_heads * L.head_dim),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel() if workspace is not None else 0,
        _stream(stream)), "kvs_append_sparse_decode_attn")


def kvs_select_topk_ex(layout: Layout, q, summaries, seq_lens, k: int, opts: SelectOpts | None,
                       append: AppendArgs | None, sel, bounds_out, workspace, stream=None) -> None:
    L = layout
    co = _opts_struct(L, opts)
    ca = _append_struct(L, append) if append is not None else None
    ws = _ptr(workspace, "workspace", torch.uint8)
    _check(_lib.kvs_select_topk_ex(
        ctypes.byref(L.c()),
        _ptr(q, "q", _TORCH_OF[L.q_dtype], L.num_seqs * L.num_q_heads * L.head_dim),
        _ptr(summaries, "summaries", L.summary_dtype_of(_kind(opts)), L.summary_numel(_kind(opts))),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        int(k),
        ctypes.byref(co) if co is not None else None,
        ctypes.byref(ca) if ca is not None else None,
        _ptr(sel, "sel", torch.int32, L.num_seqs * L.num_kv_heads * k),
        _ptr(bounds_out, "bounds_out", torch.float64, L.num_seqs * L.num_kv_heads * L.max_blocks),
        ws, workspace.numel() if workspace is not None else 0,
        _stream(stream)), "kvs_select_topk_ex")


def _opts_struct(L: Layout, opts: SelectOpts | None):
    if opts is None:
        return None
    return _CSelectOpts(int(opts.recent_blocks), 1 if opts.use_ema else 0, float(opts.ema_alpha),
                        _ptr(opts.ema_state, "ema_state", torch.float64, L.num_seqs * L.num_kv_heads * L.max_blocks),
                        int(opts.summary_kind), 1 if opts.accumulate else 0)


def _kind(opts: SelectOpts | None) -> int:
    return 0 if opts is None else int(opts.summary_kind)


def kvs_score_blocks(layout: Layout, q, summaries, seq_lens, opts: SelectOpts | None, append: AppendArgs | None,
                     scores, bounds_out, stream=None) -> None:
    L = layout
    co = _opts_struct(L, opts)
    ca = _append_struct(L, append) if append is not None else None
    n = L.num_seqs * L.num_kv_heads * L.max_blocks
    _check(_lib.kvs_score_blocks(
        ctypes.byref(L.c()),
        _ptr(q, "q", _TORCH_OF[L.q_dtype], L.num_seqs * L.num_q_heads * L.head_dim),
        _ptr(summaries, "summaries", L.summary_dtype_of(_kind(opts)), L.summary_numel(_kind(opts))),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        ctypes.byref(co) if co is not None else None,
        ctypes.byref(ca) if ca is not None else None,
        _ptr(scores, "scores", torch.float64, n),
        _ptr(bounds_out, "bounds_out", torch.float64, n),
        _stream(stream)), "kvs_score_blocks")


def kvs_select_attn(layout: Layout, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, scores,
                    k: int, recent_blocks: int, sel, sm_scale: float, out, workspace, stream=None) -> None:
    L = layout
    tile = L.num_kv_heads * L.block_size * L.head_dim
    qg = L.quant_group
    sc_n = L.num_pages * tile // qg if qg else None
    _check(_lib.kvs_select_attn(
        ctypes.byref(L.c()),
        _ptr(q, "q", _TORCH_OF[L.q_dtype], L.num_seqs * L.num_q_heads * L.head_dim),
        _ptr(k_pool, "k_pool", _pool_dtype(L), L.num_pages * tile),
        _ptr(v_pool, "v_pool", _pool_dtype(L), L.num_pages * tile),
        _ptr(k_scales, "k_scales", torch.float32, sc_n),
        _ptr(v_scales, "v_scales", torch.float32, sc_n),
        _ptr(block_table, "block_table", torch.int32, L.num_seqs * L.max_blocks),
        _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
        _ptr(scores, "scores", torch.float64, L.num_seqs * L.num_kv_heads * L.max_blocks),
        int(k), int(recent_blocks),
        _ptr(sel, "sel", torch.int32, L.num_seqs * L.num_kv_heads * k),
        float(sm_scale),
        _ptr(out, "out", torch.float32, L.num_seqs * L.num_q_heads * L.head_dim),
        _ptr(workspace, "workspace", torch.uint8),
        workspace.numel() if workspace is not None else 0,
        _stream(stream)), "kvs_select_attn")


def _attn_args(L: Layout, table_kind: int, q, k_pool, v_pool, k_scales, v_scales, table, seq_lens, sel, k: int,
               sm_scale: float, out) -> list:
    """The checked arguments shared by the two attention entry points, from
    table_kind through out."""
    if table_kind == KVS_TABLE_HOT:
        tile = L.block_size * L.head_dim
        tbl_n = L.num_seqs * L.num_kv_heads * L.max_blocks
    else:
        tile = L.num_kv_heads * L.block_size * L.head_dim
        tbl_n = L.num_seqs * L.max_blocks
    qg = L.quant_group
    sc_n = L.num_pages * tile // qg if qg else None
    return [int(table_kind),
            _ptr(q, "q", _TORCH_OF[L.q_dtype], L.num_seqs * L.num_q_heads * L.head_dim),
            _ptr(k_pool, "k_pool", _pool_dtype(L), L.num_pages * tile),
            _ptr(v_pool, "v_pool", _pool_dtype(L), L.num_pages * tile),
            _ptr(k_scales, "k_scales", torch.float32, sc_n),
            _ptr(v_scales, "v_scales", torch.float32, sc_n),
            _ptr(table, "table", torch.int32, tbl_n),
            _ptr(seq_lens, "seq_lens", torch.int32, L.num_seqs),
            _ptr(sel, "sel", torch.int32, L.num_seqs * L.num_kv_heads * k),
            int(k), float(sm_scale),
            _ptr(out, "out", torch.float32, L.num_seqs * L.num_q_heads * L.head_dim)]


def kvs_sparse_decode_attn(layout: Layout, table_kind: int, q, k_pool, v_pool, k_scales, v_scales,
                           table, seq_lens, sel, k: int, sm_scale: float, out, workspace,
                           stream=None) -> None:
    L = layout
    args = _attn_args(L, table_kind, q, k_pool, v_pool, k_scales, v_scales, table, seq_lens, sel, k, sm_scale, out)
    _check(_lib.kvs_sparse_decode_attn(
        ctypes.byref(L.c()), *args,
        _ptr(workspace, "workspace", torch.uint8),
        workspace.numel() if workspace is not None else 0,
        _stream(stream)), "kvs_sparse_decode_attn")


def kvs_sparse_decode_attn_noalloc(layout: Layout, table_kind: int, q, k_pool, v_pool, k_scales, v_scales,
                                   table, seq_lens, sel, k: int, sm_scale: float, out, stream=None) -> None:
    L = layout
    args = _attn_args(L, table_kind, q, k_pool, v_pool, k_scales, v_scales, table, seq_lens, sel, k, sm_scale, out)
    _check(_lib.kvs_sparse_decode_attn_noalloc(ctypes.byref(L.c()), *args, _stream(stream)),
           "kvs_sparse_decode_attn_noalloc")


def kvs_hot_lookup_swapin(layout: Layout, sel, k: int, num_slots: int, step: int, page_table,
                          slot_owner, slot_stamp, host_k, host_v, host_k_scales, host_v_scales,
                          hot_k, hot_v, hot_k_scales, hot_v_scales, miss_list, miss_count,
                          stream=None, live: HotLive | None = None) -> None:
    L = layout
    units = L.num_seqs * L.num_kv_heads
    tile = L.block_size * L.head_dim
    qg = L.quant_group
    host_n = units * L.max_blocks * tile
    hot_n = units * num_slots * tile
    _check(_lib.kvs_hot_lookup_swapin(
        ctypes.byref(L.c()),
        _ptr(sel, "sel", torch.int32, units * k), int(k), int(num_slots), int(step),
        _ptr(page_table, "page_table", torch.int32, units * L.max_blocks),
        _ptr(slot_owner, "slot_owner", torch.int32, units * num_slots),
        _ptr(slot_stamp, "slot_stamp", torch.int64, units * num_slots),
        _ptr(host_k, "host_k", _pool_dtype(L), host_n, device=False, pinned=True),
        _ptr(host_v, "host_v", _pool_dtype(L), host_n, device=False, pinned=True),
        _ptr(host_k_scales, "host_k_scales", torch.float32, host_n // qg if qg else None, device=False, pinned=True),
        _ptr(host_v_scales, "host_v_scales", torch.float32, host_n // qg if qg else None, device=False, pinned=True),
        _ptr(hot_k, "hot_k", _pool_dtype(L), hot_n),
        _ptr(hot_v, "hot_v", _pool_dtype(L), hot_n),
        _ptr(hot_k_scales, "hot_k_scales", torch.float32, hot_n // qg if qg else None),
        _ptr(hot_v_scales, "hot_v_scales", torch.float32, hot_n // qg if qg else None),
        _ptr(miss_list, "miss_list", torch.int32, units * k),
        _ptr(miss_count, "miss_count", torch.int32, units),
        _live_struct(L, live),
        _stream(stream)), "kvs_hot_lookup_swapin")


def kvs_hot_lookup(layout: Layout, sel, k: int, num_slots: int, step: int, page_table, slot_owner, slot_stamp,
                   miss_list, miss_count, stream=None) -> None:
    L = layout
    units = L.num_seqs * L.num_kv_heads
    _check(_lib.kvs_hot_lookup(
        ctypes.byref(L.c()),
        _ptr(sel, "sel", torch.int32, units * k), int(k), int(num_slots), int(step),
        _ptr(page_table, "page_table", torch.int32, units * L.max_blocks),
        _ptr(slot_owner, "slot_owner", torch.int32, units * num_slots),
        _ptr(slot_stamp, "slot_stamp", torch.int64, units * num_slots),
        _ptr(miss_list, "miss_list", torch.int32, units * k),
        _ptr(miss_count, "miss_count", torch.int32, units),
        _stream(stream)), "kvs_hot_lookup")


def kvs_hot_swapin(layout: Layout, k: int, num_slots: int, page_table, miss_list, miss_count, host_k, host_v,
                   host_k_scales, host_v_scales, hot_k, hot_v, hot_k_scales, hot_v_scales, stream=None,
                   live: HotLive | None = None) -> None:
    L = layout
    units = L.num_seqs * L.num_kv_heads
    tile = L.block_size * L.head_dim
    qg = L.quant_group
    host_n = units * L.max_blocks * tile
    hot_n = units * num_slots * tile
    _check(_lib.kvs_hot_swapin(
        ctypes.byref(L.c()), int(k), int(num_slots),
        _ptr(page_table, "page_table", torch.int32, units * L.max_blocks),
        _ptr(miss_list, "miss_list", torch.int32, units * k),
        _ptr(miss_count, "miss_count", torch.int32, units),
        _ptr(host_k, "host_k", _pool_dtype(L), host_n, device=False, pinned=True),
        _ptr(host_v, "host_v", _pool_dtype(L), host_n, device=False, pinned=True),
        _ptr(host_k_scales, "host_k_scales", torch.float32, host_n // qg if qg else None, device=False, pinned=True),
        _ptr(host_v_scales, "host_v_scales", torch.float32, host_n // qg if qg else None, device=False, pinned=True),
        _ptr(hot_k, "hot_k", _pool_dtype(L), hot_n),
        _ptr(hot_v, "hot_v", _pool_dtype(L), hot_n),
        _ptr(hot_k_scales, "hot_k_scales", torch.float32, hot_n // qg if qg else None),
        _ptr(hot_v_scales, "hot_v_scales", torch.float32, hot_n // qg if qg else None),
        _live_struct(L, live),
        _stream(stream)), "kvs_hot_swapin")


def kvs_select_workspace_size(layout: Layout, k: int) -> int:
    return int(_lib.kvs_select_workspace_size(ctypes.byref(layout.c()), int(k)))


def kvs_attn_workspace_size(layout: Layout, k: int) -> int:
    return int(_lib.kvs_attn_workspace_size(ctypes.byref(layout.c()), int(k)))


def kvs_select_uses_matrix_cores(layout: Layout, k: int) -> bool:
    return bool(_lib.kvs_select_uses_matrix_cores(ctypes.byref(layout.c()), int(k)))


def kvs_attn_num_splits(layout: Layout, k: int) -> int:
    return int(_lib.kvs_attn_num_splits(ctypes.byref(layout.c()), int(k)))


def kvs_device_errors(clear: bool = True, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(_lib.kvs_device_errors(ctypes.byref(flags), 1 if clear else 0, _stream(stream)),
           "kvs_device_errors")
    return int(flags.value)


def kvs_status_string(status: int) -> str:
    return _lib.kvs_status_string(int(status)).decode()


def kvs_last_error() -> str:
    return _lib.kvs_last_error().decode()


def kvs_abi_version() -> int:
    return int(_lib.kvs_abi_version())
