"""Plain fp64 CPU oracle for query-aware block-sparse decode attention.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; the product package never
does.  The arithmetic lives in ``oracle.c`` (plain C, one thread, fp64); this
module only compiles it and marshals numpy arrays through ctypes.

Every function mirrors one in ``oracle.h``; the page citations are there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

KV_F32, KV_BF16, KV_E4M3 = 0, 1, 2
OR_OK, OR_EARG, OR_ERANGE, OR_EORDER, OR_ECAP = 0, 1, 2, 3, 4


class OracleError(RuntimeError):
    pass


# A process may load another build of the same source instead (the
# sanitizer build below), named by this environment variable.
_LIB_ENV = "ORACLE_LIB"

SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False, out: str | None = None) -> str:
    """Compile liboracle.so with gcc (no fast-math, no FP contraction).  With
    sanitize, an AddressSanitizer + UndefinedBehaviorSanitizer build (same
    arithmetic flags) goes to `out` instead; a process loads it by naming it
    in ORACLE_LIB, with gcc's libasan preloaded."""
    target = out if out else _LIB
    if force or not os.path.exists(target):
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", *(SANITIZE_FLAGS if sanitize else []),
               "-o", target + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(target + ".tmp", target)
    return target


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "Hq", "Hkv", "D", "S", "max_blocks", "num_pages", "kv_dtype", "quant_group")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get(_LIB_ENV) or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        LP = ctypes.POINTER(_Layout)
        sig = {
            "or_bf16_to_f64": (f64, [ctypes.c_uint16]),
            "or_e4m3_to_f64": (f64, [ctypes.c_uint8]),
            "or_e4m3_scaled": (ctypes.c_float, [ctypes.c_uint8, ctypes.c_float]),
            "or_kv_bytes_per_token": (i64, [i32, i32, i32, i32]),
            "or_summaries": (ctypes.c_int, [LP, P, P, P, P, P, i32, P]),
            "or_bounds": (ctypes.c_int, [LP, P, P, P, P, P]),
            "or_select": (ctypes.c_int, [LP, P, P, i32, P]),
            "or_select_window": (ctypes.c_int, [LP, P, P, i32, i32, P]),
            "or_ema_scores": (ctypes.c_int, [LP, P, P, f64, P, P]),
            "or_fuse_scores": (ctypes.c_int, [LP, P, i32, P, P]),
            "or_append_token": (ctypes.c_int, [LP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]),
            "or_summaries_mean": (ctypes.c_int, [LP, P, P, P, P, P, i32, P]),
            "or_mean_scores": (ctypes.c_int, [LP, P, P, P, P, P]),
            "or_sparse_attn": (ctypes.c_int, [LP, P, P, P, P, P, P, P, P, i32, f64, P]),
            "or_dense_attn": (ctypes.c_int, [LP, P, P, P, P, P, P, P, f64, P]),
            "or_hot_step": (ctypes.c_int, [i32, i32, i32, i64, i32, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != OR_OK:
        raise OracleError(f"{what} returned oracle error {rc}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """Contiguous numpy copy/view with the given dtype (no value change)."""
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class Layout:
    """Shapes of one problem (see oracle.h for the meaning of each field)."""

    def __init__(self, B, Hq, Hkv, D, S, max_blocks, num_pages, kv_dtype, quant_group=0):
        self.B, self.Hq, self.Hkv, self.D, self.S = B, Hq, Hkv, D, S
        self.max_blocks, self.num_pages = max_blocks, num_pages
        self.kv_dtype, self.quant_group = kv_dtype, quant_group

    def c(self):
        return _Layout(self.B, self.Hq, self.Hkv, self.D, self.S, self.max_blocks,
                       self.num_pages, self.kv_dtype, self.quant_group)


_POOL_DTYPE = {KV_F32: np.float32, KV_BF16: np.uint16, KV_E4M3: np.uint8}


def _pool(L: Layout, a):
    a = np.ascontiguousarray(a)
    want = _POOL_DTYPE[L.kv_dtype]
    if a.dtype != want:
        raise TypeError(f"pool dtype {a.dtype}, expected {want} for kv_dtype {L.kv_dtype}")
    return a


def bf16_to_f64(bits: int) -> float:
    return lib().or_bf16_to_f64(bits)


def e4m3_to_f64(code: int) -> float:
    return lib().or_e4m3_to_f64(code)


def e4m3_scaled(code: int, scale: float) -> float:
    return lib().or_e4m3_scaled(code, scale)


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    return lib().or_kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem)


def summaries(L: Layout, k_pool, k_scales, block_table, seq_lens, first_block=None,
              num_rebuild=None, out=None):
    """Returns (or fills) the [B][Hkv][max_blocks][2][D] fp64 min/max table."""
    kp = _pool(L, k_pool)
    ks = _c(k_scales, np.float32)
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    fb = _c(first_block, np.int32)
    if num_rebuild is None:
        num_rebuild = L.max_blocks
    if out is None:
        out = np.full((L.B, L.Hkv, L.max_blocks, 2, L.D), np.nan, dtype=np.float64)
    assert out.dtype == np.float64 and out.flags.c_contiguous
    _check(lib().or_summaries(ctypes.byref(L.c()), _ptr(kp), _ptr(ks), _ptr(bt), _ptr(sl),
                              _ptr(fb), num_rebuild, _ptr(out)), "or_summaries")
    return out


def bounds(L: Layout, q, summ, seq_lens, want_u=False):
    """Returns W [B][Hkv][max_blocks] (and U [B][Hq][max_blocks] if asked)."""
    q = _c(q, np.float64)
    summ = _c(summ, np.float64)
    sl = _c(seq_lens, np.int32)
    W = np.empty((L.B, L.Hkv, L.max_blocks), dtype=np.float64)
    U = np.empty((L.B, L.Hq, L.max_blocks), dtype=np.float64) if want_u else None
    _check(lib().or_bounds(ctypes.byref(L.c()), _ptr(q), _ptr(summ), _ptr(sl), _ptr(U), _ptr(W)),
           "or_bounds")
    return (W, U) if want_u else W


def summaries_mean(L: Layout, k_pool, k_scales, block_table, seq_lens, first_block=None,
                   num_rebuild=None, out=None):
    """Returns (or fills) the [B][Hkv][max_blocks][D] fp32 mean table."""
    kp = _pool(L, k_pool)
    ks = _c(k_scales, np.float32)
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    fb = _c(first_block, np.int32)
    if num_rebuild is None:
        num_rebuild = L.max_blocks
    if out is None:
        out = np.full((L.B, L.Hkv, L.max_blocks, L.D), np.nan, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous
    _check(lib().or_summaries_mean(ctypes.byref(L.c()), _ptr(kp), _ptr(ks), _ptr(bt), _ptr(sl), _ptr(fb),
                                   num_rebuild, _ptr(out)), "or_summaries_mean")
    return out


def mean_scores(L: Layout, q, mean, seq_lens, want_u=False):
    """Returns W [B][Hkv][max_blocks] (and U [B][Hq][max_blocks] if asked)."""
    q = _c(q, np.float64)
    mean = _c(mean, np.float32)
    sl = _c(seq_lens, np.int32)
    W = np.empty((L.B, L.Hkv, L.max_blocks), dtype=np.float64)
    U = np.empty((L.B, L.Hq, L.max_blocks), dtype=np.float64) if want_u else None
    _check(lib().or_mean_scores(ctypes.byref(L.c()), _ptr(q), _ptr(mean), _ptr(sl), _ptr(U), _ptr(W)),
           "or_mean_scores")
    return (W, U) if want_u else W


def select(L: Layout, W, seq_lens, k):
    W = _c(W, np.float64)
    sl = _c(seq_lens, np.int32)
    sel = np.empty((L.B, L.Hkv, k), dtype=np.int32)
    _check(lib().or_select(ctypes.byref(L.c()), _ptr(W), _ptr(sl), k, _ptr(sel)), "or_select")
    return sel


def select_window(L: Layout, W, seq_lens, k, recent):
    W = _c(W, np.float64)
    sl = _c(seq_lens, np.int32)
    sel = np.empty((L.B, L.Hkv, k), dtype=np.int32)
    _check(lib().or_select_window(ctypes.byref(L.c()), _ptr(W), _ptr(sl), k, recent, _ptr(sel)),
           "or_select_window")
    return sel


def ema_scores(L: Layout, W, seq_lens, alpha, state):
    """Smoothed scores; `state` ([B][Hkv][max_blocks] fp64, NaN = no history)
    is updated in place."""
    W = _c(W, np.float64)
    sl = _c(seq_lens, np.int32)
    assert state.dtype == np.float64 and state.flags.c_contiguous
    out = np.empty((L.B, L.Hkv, L.max_blocks), dtype=np.float64)
    _check(lib().or_ema_scores(ctypes.byref(L.c()), _ptr(W), _ptr(sl), float(alpha), _ptr(state),
                               _ptr(out)), "or_ema_scores")
    return out


def fuse_scores(L: Layout, W_layers, seq_lens):
    """Sum of several layers' scores, left to right in fp64 (-inf past each
    sequence's blocks); W_layers is a list (or [n][B][Hkv][max_blocks]
    array) of per-layer scores."""
    arrs = [np.asarray(w, dtype=np.float64) for w in W_layers]
    W = np.ascontiguousarray(np.stack(arrs)) if arrs else np.zeros((0, L.B, L.Hkv, L.max_blocks))
    sl = _c(seq_lens, np.int32)
    out = np.empty((L.B, L.Hkv, L.max_blocks), dtype=np.float64)
    _check(lib().or_fuse_scores(ctypes.byref(L.c()), _ptr(W), W.shape[0], _ptr(sl), _ptr(out)),
           "or_fuse_scores")
    return out


def append_token(L: Layout, k_new, v_new, k_new_scales, v_new_scales, block_table, seq_lens,
                 k_pool, v_pool, k_scales, v_scales, summ, host_k=None, host_v=None,
                 host_k_scales=None, host_v_scales=None):
    """Appends one token per sequence; pools, scales, summaries and the host
    tier (numpy, C-contiguous) are updated in place."""
    kn, vn = _pool(L, k_new), _pool(L, v_new)
    kns, vns = _c(k_new_scales, np.float32), _c(v_new_scales, np.float32)
    bt, sl = _c(block_table, np.int32), _c(seq_lens, np.int32)
    for a in (k_pool, v_pool, host_k, host_v):
        if a is not None:
            assert a.dtype == _POOL_DTYPE[L.kv_dtype] and a.flags.c_contiguous
    for a in (k_scales, v_scales, host_k_scales, host_v_scales):
        if a is not None:
            assert a.dtype == np.float32 and a.flags.c_contiguous
    assert summ.dtype == np.float64 and summ.flags.c_contiguous
    _check(lib().or_append_token(ctypes.byref(L.c()), _ptr(kn), _ptr(vn), _ptr(kns), _ptr(vns),
                                 _ptr(bt), _ptr(sl), _ptr(k_pool), _ptr(v_pool), _ptr(k_scales),
                                 _ptr(v_scales), _ptr(summ), _ptr(host_k), _ptr(host_v),
                                 _ptr(host_k_scales), _ptr(host_v_scales)), "or_append_token")


def sparse_attn(L: Layout, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, sel,
                sm_scale):
    q = _c(q, np.float64)
    kp, vp = _pool(L, k_pool), _pool(L, v_pool)
    ks, vs = _c(k_scales, np.float32), _c(v_scales, np.float32)
    bt, sl = _c(block_table, np.int32), _c(seq_lens, np.int32)
    sel = _c(sel, np.int32)
    k = sel.shape[-1]
    out = np.empty((L.B, L.Hq, L.D), dtype=np.float64)
    _check(lib().or_sparse_attn(ctypes.byref(L.c()), _ptr(q), _ptr(kp), _ptr(vp), _ptr(ks),
                                _ptr(vs), _ptr(bt), _ptr(sl), _ptr(sel), k, float(sm_scale),
                                _ptr(out)), "or_sparse_attn")
    return out


def dense_attn(L: Layout, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens,
               sm_scale):
    q = _c(q, np.float64)
    kp, vp = _pool(L, k_pool), _pool(L, v_pool)
    ks, vs = _c(k_scales, np.float32), _c(v_scales, np.float32)
    bt, sl = _c(block_table, np.int32), _c(seq_lens, np.int32)
    out = np.empty((L.B, L.Hq, L.D), dtype=np.float64)
    _check(lib().or_dense_attn(ctypes.byref(L.c()), _ptr(q), _ptr(kp), _ptr(vp), _ptr(ks),
                               _ptr(vs), _ptr(bt), _ptr(sl), float(sm_scale), _ptr(out)),
           "or_dense_attn")
    return out


def hot_step(nb, ns, step, slot_base, sel_row, pt, owner, stamp):
    """One unit's hot-buffer step; pt/owner/stamp (numpy) are updated in place.

    Returns (miss_list, miss_cnt) or raises OracleError (OR_ECAP etc.)."""
    sel_row = _c(sel_row, np.int32)
    for a, dt in ((pt, np.int32), (owner, np.int32), (stamp, np.int64)):
        assert a.dtype == dt and a.flags.c_contiguous
    k = sel_row.shape[0]
    miss = np.empty(k, dtype=np.int32)
    cnt = np.zeros(1, dtype=np.int32)
    rc = lib().or_hot_step(nb, ns, k, step, slot_base, _ptr(sel_row), _ptr(pt), _ptr(owner),
                           _ptr(stamp), _ptr(miss), _ptr(cnt))
    if rc != OR_OK:
        raise OracleError(f"or_hot_step returned oracle error {rc}")
    return miss, int(cnt[0])
