"""The C-ABI library loads, exports every entry point include/kvs.h declares,
and rejects bad host-visible arguments before touching the GPU (these calls
return during validation, so they run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvs.h")


@pytest.fixture(scope="module")
def kvs():
    lib = os.path.join(ROOT, "query_aware_sparse_kvs_amd", "libkvs.so")
    if not os.path.exists(lib):
        from query_aware_sparse_kvs_amd import build
        build.build()
    from query_aware_sparse_kvs_amd import kvs as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls_and_helpers():
    names = declared_functions()
    for n in ("kvs_build_summaries", "kvs_select_topk", "kvs_sparse_decode_attn",
              "kvs_hot_lookup_swapin", "kvs_select_workspace_size", "kvs_attn_workspace_size",
              "kvs_device_errors", "kvs_status_string", "kvs_last_error", "kvs_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(kvs):
    lib = kvs.library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in kvs.h but not exported"
    assert set(kvs.EXPORTED) == set(declared_functions())


def test_abi_version_and_status_strings(kvs):
    assert kvs.kvs_abi_version() == 6
    for st in range(5):
        assert kvs.kvs_status_string(st).startswith("KVS_")
    assert "unknown" in kvs.kvs_status_string(99)


def _layout(kvs, **kw):
    base = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=64,
                max_blocks=16, num_pages=32, q_dtype=kvs.KVS_BF16, kv_dtype=kvs.KVS_BF16,
                quant_group=0)
    base.update(kw)
    return kvs.Layout(**base)


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def _select(kvs, L, k=4, ws_bytes=1 << 20, q=FAKE, summ=FAKE):
    lib = kvs.library()
    return lib.kvs_select_topk(ctypes.byref(L.c()), q, summ, FAKE, k, FAKE, None, FAKE, ws_bytes, None)


def _attn(kvs, L, k=4, kind=0, ws_bytes=1 << 24, scale=0.1):
    lib = kvs.library()
    return lib.kvs_sparse_decode_attn(ctypes.byref(L.c()), kind, FAKE, FAKE, FAKE, None, None, FAKE,
                                      FAKE, FAKE, k, scale, FAKE, FAKE, ws_bytes, None)


def test_workspace_sizes(kvs):
    L = _layout(kvs)
    assert kvs.kvs_select_workspace_size(L, 4) >= 8 * 2 * 2 * 16
    assert kvs.kvs_select_workspace_size(L, 1) == 0  # k < 2
    n = kvs.kvs_attn_num_splits(L, 8)
    assert 1 <= n <= 8
    assert kvs.kvs_attn_workspace_size(L, 8) >= 4 * 2 * 8 * n * (128 + 2)
    assert kvs.kvs_attn_workspace_size(L, 17) == 0  # k > max_blocks
    assert kvs.kvs_attn_workspace_size(_layout(kvs, head_dim=96), 4) == 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, 2), ("head_dim", 0, 1), ("block_size", 128, 2), ("block_size", 0, 1),
    ("num_q_heads", 7, 1), ("num_q_heads", 2 * 32, 2), ("num_kv_heads", 0, 1),
    ("max_blocks", 0, 1), ("max_blocks", 9000, 2), ("num_pages", 0, 1), ("num_seqs", -1, 1),
    ("q_dtype", 2, 2), ("kv_dtype", 7, 1), ("quant_group", 32, 1),
])
def test_select_rejects_bad_layouts(kvs, field, value, status):
    L = _layout(kvs, **{field: value})
    assert _select(kvs, L) == status
    assert kvs.kvs_last_error() != ""


def test_fp8_layout_rules(kvs):
    ok = _layout(kvs, kv_dtype=kvs.KVS_FP8_E4M3, quant_group=48)
    assert _attn(kvs, ok) == kvs.KVS_ERR_UNSUPPORTED
    bad_pair = _layout(kvs, q_dtype=kvs.KVS_F32, kv_dtype=kvs.KVS_FP8_E4M3, quant_group=32)
    assert _attn(kvs, bad_pair) == kvs.KVS_ERR_UNSUPPORTED  # (fp32 q, fp8 kv) pair
    good = _layout(kvs, kv_dtype=kvs.KVS_FP8_E4M3, quant_group=32)
    assert _attn(kvs, good) == kvs.KVS_ERR_INVALID_ARG  # fp8 without scales


def test_select_argument_checks(kvs):
    L = _layout(kvs)
    assert _select(kvs, L, k=1) == kvs.KVS_ERR_INVALID_ARG
    assert _select(kvs, L, k=17) == kvs.KVS_ERR_INVALID_ARG
    assert _select(kvs, L, ws_bytes=8) == kvs.KVS_ERR_INVALID_ARG
    assert _select(kvs, L, q=None) == kvs.KVS_ERR_INVALID_ARG
    assert _select(kvs, L, summ=ctypes.c_void_p(0x100004)) == kvs.KVS_ERR_INVALID_ARG  # misaligned


def test_attention_argument_checks(kvs):
    L = _layout(kvs)
    assert _attn(kvs, L, k=0) == kvs.KVS_ERR_INVALID_ARG
    assert _attn(kvs, L, kind=2) == kvs.KVS_ERR_INVALID_ARG
    assert _attn(kvs, L, ws_bytes=16) == kvs.KVS_ERR_INVALID_ARG
    assert _attn(kvs, L, scale=float("nan")) == kvs.KVS_ERR_INVALID_ARG
    assert _attn(kvs, L, scale=float("inf")) == kvs.KVS_ERR_INVALID_ARG


def test_summaries_and_hot_argument_checks(kvs):
    lib = kvs.library()
    L = _layout(kvs)
    c = ctypes.byref(L.c())
    assert lib.kvs_build_summaries(c, FAKE, None, FAKE, FAKE, None, 17, FAKE, None) == 1
    assert lib.kvs_build_summaries(c, None, None, FAKE, FAKE, None, 1, FAKE, None) == 1
    fp8 = _layout(kvs, kv_dtype=kvs.KVS_FP8_E4M3, quant_group=32)
    assert lib.kvs_build_summaries(ctypes.byref(fp8.c()), FAKE, None, FAKE, FAKE, None, 1, FAKE, None) == 1

    def hot(k, ns, step=0):
        return lib.kvs_hot_lookup_swapin(c, FAKE, k, ns, step, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                         FAKE, FAKE, None, None, FAKE, FAKE, None, None)
    assert hot(8, 4) == kvs.KVS_ERR_CAPACITY
    assert hot(4, 5000) == kvs.KVS_ERR_UNSUPPORTED
    assert hot(0, 4) == kvs.KVS_ERR_INVALID_ARG
    assert hot(4, 4, step=-1) == kvs.KVS_ERR_INVALID_ARG


def _append_args(kvs, **kw):
    base = {n: FAKE.value for n, _ in kvs._CAppendArgs._fields_}
    for n in ("k_new_scales", "v_new_scales", "k_scales", "v_scales", "host_k", "host_v",
              "host_k_scales", "host_v_scales"):
        base[n] = None
    base.update(kw)
    return kvs._CAppendArgs(**base)


def test_append_and_select_ex_argument_checks(kvs):
    lib = kvs.library()
    L = _layout(kvs)
    c = ctypes.byref(L.c())
    ok = _append_args(kvs)
    assert lib.kvs_append_token(c, None, FAKE, FAKE, None) == kvs.KVS_ERR_INVALID_ARG
    assert lib.kvs_append_token(c, ctypes.byref(_append_args(kvs, k_new=None)), FAKE, FAKE, None) == 1
    assert lib.kvs_append_token(c, ctypes.byref(_append_args(kvs, host_k=FAKE.value)), FAKE, FAKE, None) == 1
    assert lib.kvs_append_token(c, ctypes.byref(_append_args(kvs, k_pool=0x100002)), FAKE, FAKE, None) == 1
    fp8 = _layout(kvs, kv_dtype=kvs.KVS_FP8_E4M3, quant_group=32)
    assert lib.kvs_append_token(ctypes.byref(fp8.c()), ctypes.byref(ok), FAKE, FAKE, None) == 1  # no scales

    def sel_ex(k, recent=1, ema=0, alpha=0.7, state=FAKE.value, app=None, kind=0, acc=0):
        o = kvs._CSelectOpts(recent, ema, alpha, state, kind, acc)
        return lib.kvs_select_topk_ex(c, FAKE, FAKE, FAKE, k, ctypes.byref(o),
                                      ctypes.byref(app) if app is not None else None,
                                      FAKE, None, FAKE, 1 << 20, None)
    assert sel_ex(4, recent=0) == kvs.KVS_ERR_INVALID_ARG
    assert sel_ex(4, recent=4) == kvs.KVS_ERR_INVALID_ARG  # k < recent + 1
    assert sel_ex(4, ema=1, alpha=1.5) == kvs.KVS_ERR_INVALID_ARG
    assert sel_ex(4, ema=1, state=None) == kvs.KVS_ERR_INVALID_ARG
    assert sel_ex(4, ema=1, state=0x100004) == kvs.KVS_ERR_INVALID_ARG  # misaligned state
    assert sel_ex(4, app=_append_args(kvs, v_new=None)) == kvs.KVS_ERR_INVALID_ARG
    assert sel_ex(4, kind=2) == kvs.KVS_ERR_INVALID_ARG
    assert sel_ex(4, acc=1) == kvs.KVS_ERR_INVALID_ARG  # accumulation is for kvs_score_blocks
    assert lib.kvs_build_summaries_ex(c, 5, FAKE, None, FAKE, FAKE, None, 1, FAKE, None) == kvs.KVS_ERR_INVALID_ARG


def test_noalloc_attention_argument_checks(kvs):
    """The allocation-free attention entry point validates like the one with
    a workspace, before it looks up its device array."""
    lib = kvs.library()
    L = _layout(kvs)
    c = ctypes.byref(L.c())

    def na(k=4, kind=0, scale=0.1, out=FAKE, layout=c):
        return lib.kvs_sparse_decode_attn_noalloc(layout, kind, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                                                  k, scale, out, None)
    assert na(k=0) == kvs.KVS_ERR_INVALID_ARG
    assert na(k=17) == kvs.KVS_ERR_INVALID_ARG
    assert na(kind=2) == kvs.KVS_ERR_INVALID_ARG
    assert na(scale=float("nan")) == kvs.KVS_ERR_INVALID_ARG
    assert na(out=None) == kvs.KVS_ERR_INVALID_ARG
    assert na(layout=ctypes.byref(_layout(kvs, head_dim=96).c())) == kvs.KVS_ERR_UNSUPPORTED


def test_attention_workspace_bounded_for_every_split_count(kvs):
    """Several splits per unit only while sequences x KV heads < 256, so the
    split partials of every accepted layout fit the no-allocation entry
    point's device array (KVS_NOALLOC_SCRATCH_BYTES = 8 MiB)."""
    worst = 0
    for B in (1, 2, 3, 5, 8, 16, 31, 32, 63, 64, 100, 127, 128, 255, 256, 1024):
        for Hkv in (1, 2, 4, 8):
            for G in (1, 4, 16):
                for k in (1, 2, 7, 64, 128, 512):
                    L = _layout(kvs, num_seqs=B, num_kv_heads=Hkv, num_q_heads=G * Hkv, max_blocks=512)
                    n = kvs.kvs_attn_num_splits(L, k)
                    ws = kvs.kvs_attn_workspace_size(L, k)
                    if n == 1:
                        assert ws == 256
                    else:
                        assert B * Hkv < 256
                    worst = max(worst, ws)
    assert worst <= (17 << 18)  # 4.25 MiB


def test_split_hot_calls_argument_checks(kvs):
    """kvs_hot_lookup and kvs_hot_swapin validate like kvs_hot_lookup_swapin,
    each needing only its own half's buffers."""
    lib = kvs.library()
    L = _layout(kvs)
    c = ctypes.byref(L.c())

    def look(k=4, ns=4, step=0, sel=FAKE, owner=FAKE):
        return lib.kvs_hot_lookup(c, sel, k, ns, step, FAKE, owner, FAKE, FAKE, FAKE, None)

    def copy(k=4, ns=4, host_k=FAKE, hot_v=FAKE, layout=c, live=None):
        return lib.kvs_hot_swapin(layout, k, ns, FAKE, FAKE, FAKE, host_k, FAKE, None, None, FAKE, hot_v,
                                  None, None, live, None)
    assert look(k=8, ns=4) == kvs.KVS_ERR_CAPACITY
    assert look(ns=5000) == kvs.KVS_ERR_UNSUPPORTED
    assert look(k=0) == kvs.KVS_ERR_INVALID_ARG
    assert look(step=-1) == kvs.KVS_ERR_INVALID_ARG
    assert look(sel=None) == kvs.KVS_ERR_INVALID_ARG
    assert look(owner=None) == kvs.KVS_ERR_INVALID_ARG
    assert copy(k=8, ns=4) == kvs.KVS_ERR_CAPACITY
    assert copy(host_k=None) == kvs.KVS_ERR_INVALID_ARG
    assert copy(hot_v=None) == kvs.KVS_ERR_INVALID_ARG
    assert copy(hot_v=0x100004) == kvs.KVS_ERR_INVALID_ARG  # misaligned
    fp8 = _layout(kvs, kv_dtype=kvs.KVS_FP8_E4M3, quant_group=32)
    assert copy(layout=ctypes.byref(fp8.c())) == kvs.KVS_ERR_INVALID_ARG  # fp8 without scales

    # the live cache the newest blocks come from: every pointer, aligned pools, fp8 scales
    def live(**kw):
        f = {n: FAKE.value for n, _ in kvs._CHotLive._fields_}
        f.update(k_scales=None, v_scales=None)
        f.update(kw)
        return ctypes.byref(kvs._CHotLive(**f))
    for bad in (live(k_pool=None), live(v_pool=None), live(block_table=None), live(seq_lens=None),
                live(v_pool=0x100004)):
        assert copy(live=bad) == kvs.KVS_ERR_INVALID_ARG
        assert "live" in kvs.kvs_last_error()
    fp8_hot = lambda lv: lib.kvs_hot_swapin(ctypes.byref(fp8.c()), 4, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, FAKE, FAKE, lv, None)
    assert fp8_hot(live()) == kvs.KVS_ERR_INVALID_ARG and "live" in kvs.kvs_last_error()
