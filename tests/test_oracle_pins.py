"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against what the pages or the mathematics fix:
library decoders, the worked KV arithmetic printed on the SparDA page, closed
forms of the bound (box vertices), invariants that hold exactly in floating
point, brute-force enumeration of selections, textbook attention (torch SDPA
and numpy softmax on gathered tokens), and a hand-worked hot-buffer example.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# small problem builder (numpy, random pages, poisoned unused memory)
# ---------------------------------------------------------------------------

POISON = 1.0e6


def make_problem(orc, rng, B=2, Hq=4, Hkv=2, D=8, S=4, max_blocks=6, lens=(21, 9),
                 kv_dtype=0, quant_group=0, extra_pages=3):
    """Random fp32/bf16/e4m3 paged problem.  Token slots past a sequence's
    length and pages no table row uses hold +-POISON, so a read of them
    shows up in every result."""
    lens = np.asarray(lens, dtype=np.int32)
    assert len(lens) == B
    P = B * max_blocks + extra_pages
    pages = rng.permutation(P)[: B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    x = rng.standard_normal((2, P, Hkv, S, D))
    used = np.zeros((P, S), dtype=bool)
    for b in range(B):
        for t in range(int(lens[b])):
            used[pages[b, t // S], t % S] = True
    sign = np.where(rng.random(x.shape) < 0.5, -1.0, 1.0)
    x = np.where(used[None, :, None, :, None], x, sign * POISON)
    L = orc.Layout(B, Hq, Hkv, D, S, max_blocks, P, kv_dtype, quant_group)
    prob = dict(L=L, table=pages, lens=lens, k_scales=None, v_scales=None)
    # values are drawn token-major [P][Hkv][S][D]; the V pool stores each
    # tile as runs of T = min(S, 32) tokens, each channel-major,
    # [P][Hkv][S/T][D][T] (the *_val arrays stay token-major)
    T = min(S, 32)
    tr = lambda a, n: (np.ascontiguousarray(np.swapaxes(a.reshape(P, Hkv, S // T, T, D), -1, -2))
                       if n == "v" else a)
    if kv_dtype == orc.KV_F32:
        for i, n in enumerate("kv"):
            prob[n + "_pool"] = tr(x[i].astype(np.float32), n)
            prob[n + "_val"] = x[i].astype(np.float32).astype(np.float64)
    elif kv_dtype == orc.KV_BF16:
        for i, n in enumerate("kv"):
            t = torch.from_numpy(x[i].astype(np.float32)).to(torch.bfloat16)
            prob[n + "_pool"] = tr(t.view(torch.int16).numpy().view(np.uint16).copy(), n)
            prob[n + "_val"] = t.double().numpy()
    else:
        from query_aware_sparse_kvs_amd.synth import quantize_e4m3
        xx = np.where(np.abs(x) >= POISON, np.sign(x) * 300.0, x)
        for i, n in enumerate("kv"):
            codes, scales = quantize_e4m3(torch.from_numpy(xx[i].astype(np.float32)), quant_group)
            prob[n + "_pool"] = tr(codes.numpy(), n)
            prob[n + "_scales"] = scales.numpy()
            deq = codes.view(torch.float8_e4m3fn).float().reshape(*codes.shape[:-1], D // quant_group, quant_group)
            prob[n + "_val"] = (deq * scales[..., None]).reshape(codes.shape).double().numpy()
    prob["q"] = rng.standard_normal((B, Hq, D))
    return prob


def logical(prob, which, b, g):
    """[len][D] fp64 tokens of one (sequence, KV head), gathered by numpy."""
    L = prob["L"]
    n = int(prob["lens"][b])
    t = np.arange(n)
    return prob[which + "_val"][prob["table"][b, t // L.S], g, t % L.S, :]


def nblocks(L, n):
    return (int(n) + L.S - 1) // L.S


# ---------------------------------------------------------------------------
# decoders
# ---------------------------------------------------------------------------

def test_bf16_decoder_matches_library_on_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = np.array([orc.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decoder_matches_library_and_textbook(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.e4m3_to_f64(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # OCP E4M3FN: bias 7, 3 mantissa bits, no infinities
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert got[0x38] == 1.0 and got[0x00] == 0.0 and np.signbit(got[0x80])


def test_e4m3_scaled_is_one_fp32_rounding(orc):
    rng = np.random.default_rng(0)
    for code in range(256):
        if code in (0x7F, 0xFF):
            continue
        for scale in rng.uniform(1e-3, 3.0, size=4).astype(np.float32):
            want = np.float32(np.float32(orc.e4m3_to_f64(code)) * scale)
            got = np.float32(orc.e4m3_scaled(code, float(scale)))
            assert got == want


# ---------------------------------------------------------------------------
# the page's KV arithmetic
# ---------------------------------------------------------------------------

def _golden(name):
    vals = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("=", 1))
                vals[k] = float(v)
    return vals


def test_kv_bytes_per_token_matches_page_arithmetic(orc):
    g = _golden("kv_arithmetic.txt")
    per_tok = orc.kv_bytes_per_token(int(g["layers"]), int(g["kv_heads"]), int(g["head_dim"]),
                                     int(g["bytes_per_elem"]))
    assert per_tok == g["bytes_per_token"] == 64 * 1024
    assert per_tok * g["tokens_32k"] == g["bytes_32k"]
    assert per_tok * g["tokens_128k"] == g["bytes_128k"]
    t = g["bytes_32k"] / g["bandwidth_bytes_per_s"]
    assert abs(t - g["read_time_32k_s_approx"]) / g["read_time_32k_s_approx"] < 0.1
    kept = g["kept_fraction"] * g["bytes_32k"]
    assert abs(kept - g["kept_bytes_approx"]) / g["kept_bytes_approx"] < 0.1
    assert abs(kept / g["bandwidth_bytes_per_s"] - g["kept_read_time_s_approx"]) < 0.1 * g["kept_read_time_s_approx"]


# ---------------------------------------------------------------------------
# summaries
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype,qg", [(0, 0), (1, 0), (2, 4)])
def test_summaries_are_blockwise_min_max_of_valid_tokens(orc, kv_dtype, qg):
    rng = np.random.default_rng(1 + kv_dtype)
    p = make_problem(orc, rng, kv_dtype=kv_dtype, quant_group=qg)
    L = p["L"]
    out = orc.summaries(L, p["k_pool"], p["k_scales"], p["table"], p["lens"])
    for b in range(L.B):
        for g in range(L.Hkv):
            toks = logical(p, "k", b, g)
            for j in range(nblocks(L, p["lens"][b])):
                blk = toks[j * L.S:(j + 1) * L.S]
                mn, mx = out[b, g, j, 0], out[b, g, j, 1]
                assert np.array_equal(mn, blk.min(axis=0))
                assert np.array_equal(mx, blk.max(axis=0))
                assert (blk >= mn).all() and (blk <= mx).all()
                assert np.abs(mx).max() < POISON / 2  # no token past len was read
            # blocks past nb are not written
            assert np.isnan(out[b, g, nblocks(L, p["lens"][b]):]).all()


def test_summaries_block_size_one_is_the_key_itself(orc):
    rng = np.random.default_rng(2)
    p = make_problem(orc, rng, S=1, max_blocks=7, lens=(7, 3))
    out = orc.summaries(p["L"], p["k_pool"], None, p["table"], p["lens"])
    for b in range(2):
        for g in range(2):
            toks = logical(p, "k", b, g)
            assert np.array_equal(out[b, g, : len(toks), 0], toks)
            assert np.array_equal(out[b, g, : len(toks), 1], toks)


def test_summaries_rebuild_range(orc):
    rng = np.random.default_rng(3)
    p = make_problem(orc, rng, lens=(21, 9))  # nb = 6 and 3
    L = p["L"]
    full = orc.summaries(L, p["k_pool"], None, p["table"], p["lens"])
    part = orc.summaries(L, p["k_pool"], None, p["table"], p["lens"],
                         first_block=np.array([4, 1], np.int32), num_rebuild=5)
    assert np.array_equal(part[0, :, 4:6], full[0, :, 4:6]) and np.isnan(part[0, :, :4]).all()
    assert np.array_equal(part[1, :, 1:3], full[1, :, 1:3]) and np.isnan(part[1, :, :1]).all()
    assert np.isnan(part[1, :, 3:]).all()


# ---------------------------------------------------------------------------
# bounds
# ---------------------------------------------------------------------------

def _dot_ascending(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc = acc + float(x) * float(y)
    return acc


def test_bound_is_max_of_q_dot_x_over_box_vertices(orc):
    rng = np.random.default_rng(4)
    p = make_problem(orc, rng, D=8, lens=(21, 14))
    L = p["L"]
    summ = orc.summaries(L, p["k_pool"], None, p["table"], p["lens"])
    W, U = orc.bounds(L, p["q"], summ, p["lens"], want_u=True)
    G = L.Hq // L.Hkv
    for b in range(L.B):
        for h in range(L.Hq):
            g = h // G
            for j in range(nblocks(L, p["lens"][b])):
                mn, mx = summ[b, g, j, 0], summ[b, g, j, 1]
                best = max(_dot_ascending(p["q"][b, h], np.where(np.array(v), mx, mn))
                           for v in itertools.product((False, True), repeat=L.D))
                assert U[b, h, j] == best


def test_bound_dominates_every_key_of_its_block_exactly(orc):
    rng = np.random.default_rng(5)
    for kv_dtype, qg in ((0, 0), (1, 0), (2, 4)):
        p = make_problem(orc, rng, D=16, kv_dtype=kv_dtype, quant_group=qg, lens=(23, 17))
        L = p["L"]
        summ = orc.summaries(L, p["k_pool"], p["k_scales"], p["table"], p["lens"])
        W, U = orc.bounds(L, p["q"], summ, p["lens"], want_u=True)
        G = L.Hq // L.Hkv
        for b in range(L.B):
            for h in range(L.Hq):
                toks = logical(p, "k", b, h // G)
                for t in range(len(toks)):
                    assert U[b, h, t // L.S] >= _dot_ascending(p["q"][b, h], toks[t])


def test_bound_of_single_token_block_is_the_dot_product(orc):
    rng = np.random.default_rng(6)
    p = make_problem(orc, rng, D=16, lens=(17, 5))  # last block of each has 1 token
    L = p["L"]
    summ = orc.summaries(L, p["k_pool"], None, p["table"], p["lens"])
    W, U = orc.bounds(L, p["q"], summ, p["lens"], want_u=True)
    G = L.Hq // L.Hkv
    for b, n in enumerate(p["lens"]):
        j = (int(n) - 1) // L.S
        for h in range(L.Hq):
            tok = logical(p, "k", b, h // G)[n - 1]
            assert U[b, h, j] == _dot_ascending(p["q"][b, h], tok)


def test_group_score_is_max_over_the_groups_heads(orc):
    rng = np.random.default_rng(7)
    p = make_problem(orc, rng, Hq=8, Hkv=2, lens=(21, 9))
    L = p["L"]
    summ = orc.summaries(L, p["k_pool"], None, p["table"], p["lens"])
    W, U = orc.bounds(L, p["q"], summ, p["lens"], want_u=True)
    G = 4
    for b in range(L.B):
        nb = nblocks(L, p["lens"][b])
        for g in range(L.Hkv):
            assert np.array_equal(W[b, g, :nb], U[b, g * G:(g + 1) * G, :nb].max(axis=0))
            assert np.isneginf(W[b, g, nb:]).all()
    # changing query head 5 (group 1) moves only group 1's scores
    q2 = p["q"].copy()
    q2[:, 5] *= -3.0
    W2 = orc.bounds(L, q2, summ, p["lens"])
    assert np.array_equal(W2[:, 0], W[:, 0]) and not np.array_equal(W2[:, 1], W[:, 1])


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _brute_force_select(w, nb, k):
    if nb <= k:
        return list(range(nb))
    mid = list(range(1, nb - 1))
    key = lambda j: (w[j], -j)  # larger is better
    winners = []
    for T in itertools.combinations(mid, k - 2):
        rest = [j for j in mid if j not in T]
        if not T or not rest or min(key(j) for j in T) > max(key(j) for j in rest):
            winners.append(T)
    assert len(winners) == 1
    return sorted([0, nb - 1, *winners[0]])


def _lay(orc, B, Hkv, max_blocks, S=4):
    return orc.Layout(B, Hkv, Hkv, 4, S, max_blocks, B * max_blocks, 0, 0)


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_subset_enumeration(orc, seed):
    rng = np.random.default_rng(100 + seed)
    L = _lay(orc, 3, 2, 10)
    lens = np.array([40, 37, 13], np.int32)  # nb = 10, 10, 4
    W = np.round(rng.standard_normal((3, 2, 10)), 1)  # coarse values -> many exact ties
    for k in (2, 3, 5, 8, 10, 11):
        sel = orc.select(L, W, lens, k)
        for b in range(3):
            nb = nblocks(L, lens[b])
            for g in range(2):
                want = _brute_force_select(W[b, g], nb, k)
                assert list(sel[b, g, : len(want)]) == want
                assert (sel[b, g, len(want):] == -1).all()


def test_selection_special_cases(orc):
    L = _lay(orc, 4, 1, 9)
    lens = np.array([36, 4, 0, 33], np.int32)  # nb = 9, 1, 0, 9
    W = np.zeros((4, 1, 9))
    sel = orc.select(L, W, lens, 4)  # equal scores: lowest ids win
    assert list(sel[0, 0]) == [0, 1, 2, 8]
    assert list(sel[1, 0]) == [0, -1, -1, -1]
    assert list(sel[2, 0]) == [-1, -1, -1, -1]
    assert list(orc.select(L, W, lens, 2)[0, 0]) == [0, 8]
    W[0, 0] = [-5, 9, 9, 1, 2, 9, 3, 4, -7]
    assert list(orc.select(L, W, lens, 4)[0, 0]) == [0, 1, 2, 8]
    assert list(orc.select(L, W, lens, 5)[0, 0]) == [0, 1, 2, 5, 8]
    with pytest.raises(orc.OracleError):
        orc.select(L, W, lens, 1)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _softmax_attn(q, K, V, scale):
    if len(K) == 0:
        return np.zeros_like(q)
    s = scale * (K @ q)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def _all_blocks_sel(L, lens, k):
    sel = np.full((L.B, L.Hkv, k), -1, np.int32)
    for b, n in enumerate(lens):
        nb = nblocks(L, n)
        sel[b, :, :nb] = np.arange(nb)
    return sel


@pytest.mark.parametrize("S,mb,lens", [(4, 6, (22, 1)), (64, 2, (100, 33))])
@pytest.mark.parametrize("kv_dtype,qg", [(0, 0), (1, 0), (2, 4)])
def test_dense_attention_matches_sdpa_and_numpy(orc, kv_dtype, qg, S, mb, lens):
    """Also at S = 64, where a V tile is two 32-token runs."""
    rng = np.random.default_rng(8)
    p = make_problem(orc, rng, D=16, S=S, max_blocks=mb, kv_dtype=kv_dtype, quant_group=qg, lens=lens)
    L = p["L"]
    scale = 1.0 / math.sqrt(L.D)
    out = orc.dense_attn(L, p["q"], p["k_pool"], p["v_pool"], p["k_scales"], p["v_scales"],
                         p["table"], p["lens"], scale)
    G = L.Hq // L.Hkv
    for b in range(L.B):
        for h in range(L.Hq):
            K, V = logical(p, "k", b, h // G), logical(p, "v", b, h // G)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(p["q"][b, h][None, None]), torch.from_numpy(K)[None],
                torch.from_numpy(V)[None]).numpy()[0, 0]
            np.testing.assert_allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(out[b, h], _softmax_attn(p["q"][b, h], K, V, scale),
                                       rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kv_dtype,qg", [(0, 0), (1, 0), (2, 4)])
def test_sparse_attention_over_all_blocks_equals_dense(orc, kv_dtype, qg):
    rng = np.random.default_rng(9)
    p = make_problem(orc, rng, D=16, kv_dtype=kv_dtype, quant_group=qg, lens=(23, 8))
    L = p["L"]
    args = (p["k_pool"], p["v_pool"], p["k_scales"], p["v_scales"], p["table"], p["lens"])
    dense = orc.dense_attn(L, p["q"], *args, 0.3)
    for k in (6, 9):
        sparse = orc.sparse_attn(L, p["q"], *args, _all_blocks_sel(L, p["lens"], k), 0.3)
        np.testing.assert_allclose(sparse, dense, rtol=1e-12, atol=1e-14)


def test_sparse_attention_is_softmax_over_the_selected_tokens(orc):
    rng = np.random.default_rng(10)
    p = make_problem(orc, rng, D=16, max_blocks=8, lens=(30, 19))
    L = p["L"]
    sel = np.array([[[0, 3, 7, -1], [1, 2, -1, -1]], [[0, 4, -1, -1], [-1, -1, -1, -1]]], np.int32)
    out = orc.sparse_attn(L, p["q"], p["k_pool"], p["v_pool"], None, None, p["table"], p["lens"],
                          sel, 0.25)
    G = L.Hq // L.Hkv
    for b in range(L.B):
        for h in range(L.Hq):
            g = h // G
            toks = [t for j in sel[b, g] if j >= 0 for t in range(j * L.S, min((j + 1) * L.S, p["lens"][b]))]
            K, V = logical(p, "k", b, g)[toks], logical(p, "v", b, g)[toks]
            np.testing.assert_allclose(out[b, h], _softmax_attn(p["q"][b, h], K, V, 0.25),
                                       rtol=1e-12, atol=1e-14)
    assert (out[1, 2:] == 0).all()  # empty selection -> zero row


def test_attention_of_uniform_values_is_that_value(orc):
    rng = np.random.default_rng(11)
    p = make_problem(orc, rng, D=16, lens=(21, 9))
    row = rng.standard_normal(16).astype(np.float32)
    p["v_pool"][:] = row[:, None]  # channel-major runs: V[run][c][t] = row[c]
    L = p["L"]
    sel = np.array([[[0, 2, 5, -1], [1, 5, -1, -1]], [[0, 2, -1, -1], [1, -1, -1, -1]]], np.int32)
    out = orc.sparse_attn(L, p["q"], p["k_pool"], p["v_pool"], None, None, p["table"], p["lens"],
                          sel, 1.0)
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), rtol=1e-13)


def test_attention_rejects_bad_selections(orc):
    rng = np.random.default_rng(12)
    p = make_problem(orc, rng, lens=(21, 9))
    L = p["L"]
    base = _all_blocks_sel(L, p["lens"], 6)
    args = (p["k_pool"], p["v_pool"], None, None, p["table"], p["lens"])
    for bad in ([3, 1, -1, -1, -1, -1], [1, 1, -1, -1, -1, -1], [0, -1, 2, -1, -1, -1],
                [0, 6, -1, -1, -1, -1]):
        sel = base.copy()
        sel[0, 0] = bad
        with pytest.raises(orc.OracleError):
            orc.sparse_attn(L, p["q"], *args, sel, 1.0)


# ---------------------------------------------------------------------------
# hot buffer step
# ---------------------------------------------------------------------------

def test_hot_step_hand_worked_example(orc):
    """ns = 3 slots, slot ids offset by slot_base = 6, 8 blocks.  Expected
    states worked out by hand from the rules (hits refresh, misses ascending,
    victims by (stamp, slot), old owner loses its slot)."""
    nb, ns, base = 8, 3, 6
    pt = np.full(nb, -1, np.int32)
    owner = np.full(ns, -1, np.int32)
    stamp = np.full(ns, -1, np.int64)

    def step(t, row):
        return orc.hot_step(nb, ns, t, base, np.array(row, np.int32), pt, owner, stamp)

    miss, m = step(0, [0, 3, 7, -1])  # empty buffer: free slots 0,1,2 in order
    assert m == 3 and list(miss) == [0, 3, 7, -1]
    assert list(owner) == [0, 3, 7] and list(stamp) == [0, 0, 0]
    assert pt[0] == 6 and pt[3] == 7 and pt[7] == 8
    miss, m = step(1, [0, 5, 7, -1])  # 0,7 hit; 5 takes slot 1 from block 3
    assert m == 1 and list(miss) == [5, -1, -1, -1]
    assert list(owner) == [0, 5, 7] and list(stamp) == [1, 1, 1] and pt[3] == -1 and pt[5] == 7
    miss, m = step(2, [0, 7, -1, -1])  # all hits
    assert m == 0 and list(stamp) == [2, 1, 2]
    miss, m = step(3, [1, 2, 7, -1])  # victims: slot 1 (stamp 1) then slot 0 (stamp 2)
    assert m == 2 and list(miss) == [1, 2, -1, -1]
    assert list(owner) == [2, 1, 7] and list(stamp) == [3, 3, 3]
    assert pt[1] == 7 and pt[2] == 6 and pt[0] == -1 and pt[5] == -1
    with pytest.raises(orc.OracleError):  # 4 blocks, 3 slots
        step(4, [0, 1, 2, 7])
    assert list(owner) == [2, 1, 7] and list(stamp) == [3, 3, 3]  # untouched
    miss, m = step(5, [3, 4, 7, -1])  # equal stamps: slot 0 before slot 1
    assert m == 2 and list(owner) == [3, 4, 7] and pt[3] == 6 and pt[4] == 7
    assert pt[1] == -1 and pt[2] == -1 and pt[7] == 8
    assert sorted(np.flatnonzero(pt >= 0)) == [3, 4, 7]


def test_hot_step_invariants_on_random_stream(orc):
    rng = np.random.default_rng(13)
    nb, ns, k, base = 20, 6, 6, 12
    pt = np.full(nb, -1, np.int32)
    owner = np.full(ns, -1, np.int32)
    stamp = np.full(ns, -1, np.int64)
    for t in range(60):
        n = int(rng.integers(0, k + 1))
        S = np.sort(rng.choice(nb, size=n, replace=False)).astype(np.int32)
        row = np.full(k, -1, np.int32)
        row[:n] = S
        pt0, owner0, stamp0 = pt.copy(), owner.copy(), stamp.copy()
        miss, m = orc.hot_step(nb, ns, t, base, row, pt, owner, stamp)
        inS = set(S.tolist())
        assert list(miss[:m]) == [j for j in S if pt0[j] < 0] and (miss[m:] == -1).all()
        for j in S:
            assert pt[j] >= 0 and owner[pt[j] - base] == j and stamp[pt[j] - base] == t
        for s in range(ns):
            if owner[s] >= 0:
                assert pt[owner[s]] == base + s
        assert (pt >= 0).sum() == (owner >= 0).sum()
        changed = [s for s in range(ns) if owner[s] != owner0[s]]
        assert len(changed) == m
        keep = [s for s in range(ns) if s not in changed and not (owner0[s] >= 0 and owner0[s] in inS)]
        for s in changed:
            assert owner0[s] < 0 or owner0[s] not in inS
            for s2 in keep:
                assert (stamp0[s], s) < (stamp0[s2], s2)
        vict = sorted(changed, key=lambda s: (stamp0[s], s))
        assert [owner[s] for s in vict] == list(miss[:m])


def test_hot_step_misses_equal_drift_when_slots_equal_k(orc):
    from query_aware_sparse_kvs_amd.synth import drift_selections
    nb, k, drift = 64, 16, 3
    rng = np.random.default_rng(14)
    sel0 = np.sort(np.concatenate([[0, nb - 1], rng.choice(np.arange(1, nb - 1), k - 2, replace=False)]))
    stream = drift_selections(sel0[None, None].astype(np.int32), nb, 12, drift, seed=7)
    pt = np.full(nb, -1, np.int32)
    owner = np.full(k, -1, np.int32)
    stamp = np.full(k, -1, np.int64)
    for t in range(stream.shape[0]):
        miss, m = orc.hot_step(nb, k, t, 0, stream[t, 0, 0], pt, owner, stamp)
        assert m == (k if t == 0 else drift)
