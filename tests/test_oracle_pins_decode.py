"""Pins of the oracle's decode-loop functions: token append with sealing to
the host tier, selection with a recent window, and score smoothing.

Each function is checked against something other than itself: the raw token
arrays the cache was filled from (numpy gathers and a numpy softmax), brute
force enumeration of the selections, and closed forms of the smoothing
recurrence.
"""
import itertools

import numpy as np
import pytest
import torch

POISON = 1.0e6


# ---------------------------------------------------------------------------
# token append and sealing
# ---------------------------------------------------------------------------

def _encode(orc, kv_dtype, x, qg):
    """Raw fp64 tokens [..., D] -> (stored elements, scales or None, fp64 values)."""
    if kv_dtype == orc.KV_F32:
        e = x.astype(np.float32)
        return e, None, e.astype(np.float64)
    if kv_dtype == orc.KV_BF16:
        t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy(), None, t.double().numpy()
    from query_aware_sparse_kvs_amd.synth import quantize_e4m3
    codes, scales = quantize_e4m3(torch.from_numpy(x.astype(np.float32)), qg)
    D = x.shape[-1]
    deq = codes.view(torch.float8_e4m3fn).float().reshape(*codes.shape[:-1], D // qg, qg)
    val = (deq * scales[..., None]).reshape(codes.shape).double().numpy()
    return codes.numpy().copy(), scales.numpy().copy(), val


def _v_token_major(a, P, Hkv, S, D):
    """[P][Hkv][S/T][D][T] V tiles -> token-major [P][Hkv][S][D] (numpy)."""
    T = min(S, 32)
    return np.swapaxes(a.reshape(P, Hkv, S // T, D, T), -1, -2).reshape(P, Hkv, S, D)


def _value(orc, kv_dtype, elems, scales, qg):
    if kv_dtype == orc.KV_F32:
        return elems.astype(np.float64)
    if kv_dtype == orc.KV_BF16:
        return torch.from_numpy(elems.view(np.int16)).view(torch.bfloat16).double().numpy()
    D = elems.shape[-1]
    deq = torch.from_numpy(elems).view(torch.float8_e4m3fn).float().reshape(*elems.shape[:-1], D // qg, qg)
    return (deq * torch.from_numpy(scales)[..., None]).reshape(elems.shape).double().numpy()


def _appended_cache(orc, kv_dtype, qg, S, lens, seed, B=3, Hkv=2, Hq=4, D=16, MB=5):
    """Fills a poisoned paged cache by appending every token one at a time
    (sequences of different lengths grow together, as in a batched decode)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    P = B * MB + 2
    pages = rng.permutation(P)[: B * MB].reshape(B, MB).astype(np.int32)
    L = orc.Layout(B, Hq, Hkv, D, S, MB, P, kv_dtype, qg)
    dt = {orc.KV_F32: np.float32, orc.KV_BF16: np.uint16, orc.KV_E4M3: np.uint8}[kv_dtype]
    fill = {orc.KV_F32: np.float32(POISON), orc.KV_BF16: np.uint16(0x4974), orc.KV_E4M3: np.uint8(0x7E)}[kv_dtype]
    kp = np.full((P, Hkv, S, D), fill, dt)
    vp = np.full((P, Hkv, S * D), fill, dt).reshape(P, Hkv, S // min(S, 32), D, min(S, 32)).copy()
    ks = vs = hks = hvs = None
    if kv_dtype == orc.KV_E4M3:
        ks = np.full((P, Hkv, S, D // qg), 7.0, np.float32)
        vs = ks.copy()
        hks = np.full((B, Hkv, MB, S, D // qg), -3.0, np.float32)
        hvs = hks.copy()
    hk = np.full((B, Hkv, MB, S, D), fill, dt)
    hv = np.full((B, Hkv, MB, S * D), fill, dt).reshape(B, Hkv, MB, S // min(S, 32), D, min(S, 32)).copy()
    summ = np.full((B, Hkv, MB, 2, D), np.nan)
    raw_k = rng.standard_normal((B, Hkv, int(lens.max()), D))
    raw_v = rng.standard_normal((B, Hkv, int(lens.max()), D))
    ek, sk, valk = _encode(orc, kv_dtype, raw_k, qg)
    ev, sv, valv = _encode(orc, kv_dtype, raw_v, qg)
    for t in range(int(lens.max())):
        grow = lens > t  # sequences still growing append token t
        cur = np.where(grow, t + 1, lens).astype(np.int32)
        # a sequence that has stopped re-appends nothing: give it length 0
        step_lens = np.where(grow, cur, 0).astype(np.int32)
        kn = np.ascontiguousarray(ek[:, :, t])
        vn = np.ascontiguousarray(ev[:, :, t])
        kns = None if sk is None else np.ascontiguousarray(sk[:, :, t])
        vns = None if sv is None else np.ascontiguousarray(sv[:, :, t])
        orc.append_token(L, kn, vn, kns, vns, pages, step_lens, kp, vp, ks, vs, summ, hk, hv, hks, hvs)
    return dict(L=L, pages=pages, lens=lens, fill=fill, kp=kp, vp=vp, ks=ks, vs=vs, hk=hk, hv=hv, hks=hks, hvs=hvs,
                summ=summ, valk=valk, valv=valv, ek=ek, ev=ev, sk=sk, sv=sv, rng=rng)


CASES = [(0, 0, 4), (1, 0, 4), (2, 4, 4), (1, 0, 64), (2, 8, 32)]


@pytest.mark.parametrize("kv_dtype,qg,S", CASES)
def test_appended_tokens_land_where_the_cache_is_read(orc, kv_dtype, qg, S):
    lens = (3 * S + 1, S, 2 * S - 1)
    c = _appended_cache(orc, kv_dtype, qg, S, lens, seed=11 + S)
    L = c["L"]
    kv = _value(orc, kv_dtype, c["kp"], c["ks"], qg)
    vv = _value(orc, kv_dtype, _v_token_major(c["vp"], L.num_pages, L.Hkv, S, L.D),
                c["vs"], qg)
    for b, n in enumerate(lens):
        t = np.arange(n)
        pg = c["pages"][b, t // S]
        for g in range(L.Hkv):
            assert np.array_equal(kv[pg, g, t % S], c["valk"][b, g, :n])
            assert np.array_equal(vv[pg, g, t % S], c["valv"][b, g, :n])
    # every slot no token was appended to still holds its fill
    used = np.zeros((L.num_pages, S), bool)
    for b, n in enumerate(lens):
        t = np.arange(n)
        used[c["pages"][b, t // S], t % S] = True
    assert (~used).any()
    vtm = _v_token_major(c["vp"], L.num_pages, L.Hkv, S, L.D)
    for p, s in zip(*np.nonzero(~used)):
        assert (c["kp"][p, :, s] == c["fill"]).all() and (vtm[p, :, s] == c["fill"]).all()


@pytest.mark.parametrize("kv_dtype,qg,S", CASES)
def test_summaries_after_appends_are_min_max_of_the_raw_tokens(orc, kv_dtype, qg, S):
    lens = (3 * S + 1, S, 2 * S - 1)
    c = _appended_cache(orc, kv_dtype, qg, S, lens, seed=23 + S)
    L = c["L"]
    for b, n in enumerate(lens):
        for j in range((n + S - 1) // S):
            blk = c["valk"][b, :, j * S: min((j + 1) * S, n)]  # [Hkv][t][D]
            assert np.array_equal(c["summ"][b, :, j, 0], blk.min(axis=1))
            assert np.array_equal(c["summ"][b, :, j, 1], blk.max(axis=1))
        assert np.isnan(c["summ"][b, :, (n + S - 1) // S:]).all()


@pytest.mark.parametrize("kv_dtype,qg,S", CASES)
def test_sealed_blocks_and_only_those_reach_the_host_tier(orc, kv_dtype, qg, S):
    lens = (3 * S + 1, S, 2 * S - 1)
    c = _appended_cache(orc, kv_dtype, qg, S, lens, seed=31 + S)
    L = c["L"]
    hk = _value(orc, kv_dtype, c["hk"], c["hks"], qg)
    hv = _value(orc, kv_dtype, _v_token_major(c["hv"].reshape(L.B * L.Hkv * L.max_blocks, 1, -1),
                                              L.B * L.Hkv * L.max_blocks, 1, S, L.D),
                c["hvs"].reshape(L.B * L.Hkv * L.max_blocks, 1, S, -1) if c["hvs"] is not None else None,
                qg).reshape(L.B, L.Hkv, L.max_blocks, S, L.D)
    for b, n in enumerate(lens):
        for j in range(L.max_blocks):
            sealed = (j + 1) * S <= n
            if sealed:
                assert np.array_equal(hk[b, :, j], c["valk"][b, :, j * S:(j + 1) * S])
                assert np.array_equal(hv[b, :, j], c["valv"][b, :, j * S:(j + 1) * S])
            else:  # never written: still the fill pattern
                assert (c["hk"][b, :, j] == c["fill"]).all() and (c["hv"][b, :, j] == c["fill"]).all()
                if c["hks"] is not None:
                    assert (c["hks"][b, :, j] == -3.0).all() and (c["hvs"][b, :, j] == -3.0).all()


@pytest.mark.parametrize("kv_dtype,qg", [(0, 0), (1, 0), (2, 4)])
def test_attention_over_the_appended_cache_is_softmax_over_the_raw_tokens(orc, kv_dtype, qg):
    S = 4
    lens = (13, 8, 1)
    c = _appended_cache(orc, kv_dtype, qg, S, lens, seed=41)
    L = c["L"]
    q = c["rng"].standard_normal((L.B, L.Hq, L.D))
    vp = c["vp"]
    out = orc.dense_attn(L, q, c["kp"], vp, c["ks"], c["vs"], c["pages"], np.asarray(lens, np.int32), 0.25)
    G = L.Hq // L.Hkv
    for b, n in enumerate(lens):
        for h in range(L.Hq):
            K = c["valk"][b, h // G, :n]
            V = c["valv"][b, h // G, :n]
            s = 0.25 * (K @ q[b, h])
            p = np.exp(s - s.max())
            np.testing.assert_allclose(out[b, h], (p @ V) / p.sum(), rtol=1e-12, atol=1e-12)


def test_append_rejects_bad_arguments(orc):
    L = orc.Layout(1, 2, 1, 8, 4, 2, 2, orc.KV_F32, 0)
    kp = np.zeros((2, 1, 4, 8), np.float32)
    vp = np.zeros((2, 1, 1, 8, 4), np.float32)
    summ = np.zeros((1, 1, 2, 2, 8))
    kn = np.zeros((1, 1, 8), np.float32)
    table = np.array([[0, 1]], np.int32)
    with pytest.raises(orc.OracleError):  # length beyond max_blocks * S
        orc.append_token(L, kn, kn, None, None, table, np.array([9], np.int32), kp, vp, None, None, summ)
    with pytest.raises(orc.OracleError):  # page out of range
        orc.append_token(L, kn, kn, None, None, np.array([[0, 5]], np.int32), np.array([5], np.int32),
                         kp, vp, None, None, summ)


# ---------------------------------------------------------------------------
# selection with a recent window
# ---------------------------------------------------------------------------

def _brute_force_window(w, nb, k, r):
    if nb <= k:
        return list(range(nb))
    forced = [0, *range(nb - r, nb)]
    mid = list(range(1, nb - r))
    key = lambda j: (w[j], -j)  # larger is better
    winners = []
    for T in itertools.combinations(mid, k - 1 - r):
        rest = [j for j in mid if j not in T]
        if not T or not rest or min(key(j) for j in T) > max(key(j) for j in rest):
            winners.append(T)
    assert len(winners) == 1
    return sorted([*forced, *winners[0]])


@pytest.mark.parametrize("seed", range(4))
def test_window_selection_matches_subset_enumeration(orc, seed):
    rng = np.random.default_rng(300 + seed)
    L = orc.Layout(3, 2, 2, 4, 4, 11, 33, 0, 0)
    lens = np.array([44, 41, 14], np.int32)  # nb = 11, 11, 4
    W = np.round(rng.standard_normal((3, 2, 11)), 1)  # coarse values -> exact ties
    for r in (1, 2, 3):
        for k in range(r + 1, 12):
            sel = orc.select_window(L, W, lens, k, r)
            for b in range(3):
                nb = (int(lens[b]) + 3) // 4
                for g in range(2):
                    want = _brute_force_window(W[b, g], nb, k, r)
                    assert list(sel[b, g, : len(want)]) == want
                    assert (sel[b, g, len(want):] == -1).all()


def test_window_selection_special_cases(orc):
    L = orc.Layout(1, 1, 1, 4, 4, 9, 9, 0, 0)
    lens = np.array([36], np.int32)  # nb = 9
    W = np.arange(9, dtype=np.float64)[None, None, :][:, :, ::-1].copy()  # block 1 best, 7 worst
    assert list(orc.select_window(L, W, lens, 4, 3)[0, 0]) == [0, 6, 7, 8]  # k = r + 1: forced only
    assert list(orc.select_window(L, W, lens, 6, 3)[0, 0]) == [0, 1, 2, 6, 7, 8]
    assert np.array_equal(orc.select_window(L, W, lens, 5, 1), orc.select(L, W, lens, 5))
    with pytest.raises(orc.OracleError):
        orc.select_window(L, W, lens, 3, 3)  # k < r + 1
    with pytest.raises(orc.OracleError):
        orc.select_window(L, W, lens, 3, 0)


# ---------------------------------------------------------------------------
# score smoothing
# ---------------------------------------------------------------------------

def test_ema_weights_the_current_step_by_alpha(orc):
    L = orc.Layout(1, 1, 1, 4, 4, 3, 3, 0, 0)
    lens = np.array([12], np.int32)
    state = np.full((1, 1, 3), np.nan)
    zero = np.zeros((1, 1, 3))
    one = np.ones((1, 1, 3))
    out = orc.ema_scores(L, zero, lens, 0.7, state)  # no history: the score itself
    assert (out == 0).all() and (state == 0).all()
    out = orc.ema_scores(L, one, lens, 0.7, state)  # 70% now, 30% history
    assert np.allclose(out, 0.7, rtol=0, atol=1e-15)
    for n in range(2, 40):  # step response 1 - 0.3^n
        out = orc.ema_scores(L, one, lens, 0.7, state)
        assert abs(out[0, 0, 0] - (1.0 - 0.3 ** n)) <= 4e-16 * n


def test_ema_limits_and_new_blocks(orc):
    L = orc.Layout(2, 1, 1, 4, 4, 4, 8, 0, 0)
    rng = np.random.default_rng(5)
    W = rng.standard_normal((2, 1, 4))
    state = rng.standard_normal((2, 1, 4))
    state[1, 0, 2] = np.nan  # block 2 of sequence 1 is new
    keep = state.copy()
    lens = np.array([16, 9], np.int32)  # nb = 4, 3
    out = orc.ema_scores(L, W, lens, 1.0, state)  # alpha 1: the current scores
    assert np.array_equal(out[0, 0], W[0, 0]) and np.array_equal(out[1, 0, :3], W[1, 0, :3])
    assert out[1, 0, 3] == -np.inf and state[1, 0, 3] == keep[1, 0, 3]  # past nb: untouched
    state = keep.copy()
    out = orc.ema_scores(L, W, lens, 0.0, state)  # alpha 0: the history
    assert np.array_equal(out[0, 0], keep[0, 0])
    assert out[1, 0, 2] == W[1, 0, 2]  # no history yet: the score itself
    with pytest.raises(orc.OracleError):
        orc.ema_scores(L, W, lens, 1.5, state)


# ---------------------------------------------------------------------------
# mean summaries
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype,qg,S", [(1, 0, 4), (1, 0, 16), (0, 0, 4), (2, 4, 4)])
def test_mean_summaries_are_the_mean_of_the_valid_tokens(orc, kv_dtype, qg, S):
    lens = (3 * S + 1, S, 2 * S - 1)
    c = _appended_cache(orc, kv_dtype, qg, S, lens, seed=51 + S)
    L = c["L"]
    m = orc.summaries_mean(L, c["kp"], c["ks"], c["pages"], np.asarray(lens, np.int32))
    for b, n in enumerate(lens):
        for j in range((n + S - 1) // S):
            blk = c["valk"][b, :, j * S: min((j + 1) * S, n)]  # [Hkv][t][D]
            # fp64 sums of these values are exact (bf16 / small fp8 values), so
            # numpy's summation order gives the same double; one fp32 rounding
            if kv_dtype != orc.KV_F32:
                want = (blk.sum(axis=1) / blk.shape[1]).astype(np.float32)
                assert np.array_equal(m[b, :, j], want)
            else:  # fp32 values: compare with the ascending-order fp64 sum
                acc = np.zeros(blk.shape[::2])
                for t in range(blk.shape[1]):
                    acc = acc + blk[:, t, :]
                assert np.array_equal(m[b, :, j], (acc / blk.shape[1]).astype(np.float32))
            # the mean lies inside the block's min/max box
            assert (m[b, :, j] >= c["summ"][b, :, j, 0]).all() and (m[b, :, j] <= c["summ"][b, :, j, 1]).all()
        assert np.isnan(m[b, :, (n + S - 1) // S:]).all()


def test_mean_of_a_single_token_block_is_the_key_and_its_score_the_dot_product(orc):
    rng = np.random.default_rng(61)
    B, Hkv, Hq, D, MB = 2, 2, 4, 16, 5
    L = orc.Layout(B, Hq, Hkv, D, 1, MB, B * MB, orc.KV_BF16, 0)
    x = torch.from_numpy(rng.standard_normal((B * MB, Hkv, 1, D)).astype(np.float32)).to(torch.bfloat16)
    kp = x.view(torch.int16).numpy().view(np.uint16).copy()
    table = np.arange(B * MB, dtype=np.int32).reshape(B, MB)
    lens = np.array([MB, 3], np.int32)
    m = orc.summaries_mean(L, kp, None, table, lens)
    kv = x.double().numpy()
    for b in range(B):
        for j in range(lens[b]):
            assert np.array_equal(m[b, :, j], kv[table[b, j], :, 0].astype(np.float32))
    q = rng.standard_normal((B, Hq, D))
    W, U = orc.mean_scores(L, q, m, lens, want_u=True)
    summ = orc.summaries(L, kp, None, table, lens)
    Wb, Ub = orc.bounds(L, q, summ, lens, want_u=True)  # S = 1: the box bound is q.k too
    for b in range(B):
        assert np.array_equal(U[b, :, :lens[b]], Ub[b, :, :lens[b]])
        assert np.array_equal(W[b, :, :lens[b]], Wb[b, :, :lens[b]])
        assert np.isneginf(W[b, :, lens[b]:]).all()


def test_mean_score_never_exceeds_the_box_bound(orc):
    """mean lies in [min, max] per channel, so each term q*mean <= max(q*min,
    q*max) and, summed in the same order, the mean score <= the bound
    (exactly, by monotone rounding)."""
    S = 8
    lens = (5 * S - 3, 2 * S, S + 1)
    c = _appended_cache(orc, orc.KV_BF16, 0, S, lens, seed=71, MB=6)
    L = c["L"]
    ln = np.asarray(lens, np.int32)
    m = orc.summaries_mean(L, c["kp"], None, c["pages"], ln)
    q = c["rng"].standard_normal((L.B, L.Hq, L.D))
    Wm, Um = orc.mean_scores(L, q, m, ln, want_u=True)
    Wb, Ub = orc.bounds(L, q, c["summ"], ln, want_u=True)
    for b, n in enumerate(lens):
        nb = (n + S - 1) // S
        assert (Um[b, :, :nb] <= Ub[b, :, :nb]).all()
        assert (Wm[b, :, :nb] <= Wb[b, :, :nb]).all()
        # and it is the dot product with the mean of the block's keys
        G = L.Hq // L.Hkv
        for h in range(L.Hq):
            for j in range(nb):
                blk = c["valk"][b, h // G, j * S: min((j + 1) * S, n)]
                est = q[b, h] @ blk.mean(axis=0)
                assert abs(Um[b, h, j] - est) <= 1e-6 * (1 + abs(est))


# ---------------------------------------------------------------------------
# cross-layer score fusion ("SparDA…" §3.1, §4.1)
# ---------------------------------------------------------------------------

def _fuse_layout(orc, B=3, Hkv=2, MB=9, S=16):
    return orc.Layout(B, 2 * Hkv, Hkv, 8, S, MB, B * MB, orc.KV_F32)


def test_fused_score_of_integer_multiples_is_their_sum(orc):
    """Layers whose scores are 1x, 2x and 4x one integer-valued base (all
    sums exact in fp64) fuse to exactly 7x the base, entry by entry: a
    dropped or repeated layer, a max instead of a sum, or a wrong layer,
    sequence or head stride gives another multiple somewhere."""
    L = _fuse_layout(orc)
    rng = np.random.default_rng(41)
    base = rng.integers(-5000, 5000, size=(L.B, L.Hkv, L.max_blocks)).astype(np.float64)
    lens = np.array([L.max_blocks * L.S, 5 * L.S - 3, 1], np.int32)
    F = orc.fuse_scores(L, [base, 2 * base, 4 * base], lens)
    for b, n in enumerate(lens):
        nb = (int(n) + L.S - 1) // L.S
        assert np.array_equal(F[b, :, :nb], 7 * base[b, :, :nb])
        assert np.isneginf(F[b, :, nb:]).all()
    # one layer: its own scores (up to nb), the selection it gives unchanged
    F1 = orc.fuse_scores(L, [base], lens)
    W = base.copy()
    for b, n in enumerate(lens):
        W[b, :, (int(n) + L.S - 1) // L.S:] = -np.inf
    assert np.array_equal(F1, W)
    assert np.array_equal(orc.select(L, F1, lens, 4), orc.select(L, W, lens, 4))


def test_fused_score_adds_left_to_right(orc):
    """fp64 addition is not associative: with a = 1, b = 2^-53, c = 2^-53 the
    left-to-right sum (a + b) + c rounds to 1 twice, a + (b + c) does not.
    The fusion adds the layers in ascending order."""
    L = _fuse_layout(orc, B=1, Hkv=1, MB=1, S=4)
    lens = np.array([4], np.int32)
    one = np.ones((1, 1, 1))
    tiny = np.full((1, 1, 1), 2.0 ** -53)
    F = orc.fuse_scores(L, [one, tiny, tiny], lens)
    assert F[0, 0, 0] == 1.0
    F = orc.fuse_scores(L, [tiny, tiny, one], lens)
    assert F[0, 0, 0] == 1.0 + 2.0 ** -52


def test_fused_selection_respects_dominance(orc):
    """A block that scores at least as high as another in every layer is
    fused at least as high: if it is a free candidate and the other one is
    selected, it is selected too."""
    L = _fuse_layout(orc, B=2, Hkv=2, MB=40, S=16)
    rng = np.random.default_rng(43)
    lens = np.array([40 * 16, 33 * 16 - 5], np.int32)
    layers = [rng.normal(size=(L.B, L.Hkv, L.max_blocks)) * 10 for _ in range(3)]
    # block 7 dominates block 20 in every layer
    for w in layers:
        w[:, :, 7] = np.maximum(w[:, :, 7], w[:, :, 20] + 0.5)
    F = orc.fuse_scores(L, layers, lens)
    assert (F[:, :, 7] >= F[:, :, 20]).all()
    for k in range(3, 30):
        sel = orc.select(L, F, lens, k)
        for b in range(L.B):
            for g in range(L.Hkv):
                s = set(sel[b, g][sel[b, g] >= 0].tolist())
                if 20 in s:
                    assert 7 in s


def test_fuse_rejects_bad_arguments(orc):
    L = _fuse_layout(orc)
    W = np.zeros((1, L.B, L.Hkv, L.max_blocks))
    with pytest.raises(orc.OracleError):
        orc.fuse_scores(L, W[:0], np.zeros(L.B, np.int32))  # no layers
    with pytest.raises(orc.OracleError):
        orc.fuse_scores(L, W, np.full(L.B, 10 ** 6, np.int32))  # length past the table
