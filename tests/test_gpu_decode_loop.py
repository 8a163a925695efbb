"""GPU parity of the decode-loop calls, through the C ABI, against the oracle
on the same seeded inputs:

  kvs_append_token     pools, fp8 scales and the host tier bit-exact,
                       summaries equal by value, over many consecutive
                       decode steps (blocks opened, filled and sealed,
                       sequences of different lengths, empty sequences)
  kvs_select_topk_ex   selections bit-exact, smoothing state bit-exact and
                       bounds bit-exact, with a recent window and score
                       smoothing over a drifting query; its fused token
                       append gives the same cache and selection as the
                       separate call
"""
import numpy as np
import pytest

from test_gpu_parity import Problem, np_pool, no_device_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env(orc):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from query_aware_sparse_kvs_amd import kvs, synth
    torch.cuda.set_device(0)
    kvs.kvs_device_errors(clear=True)

    class Env:
        pass
    e = Env()
    e.torch, e.kvs, e.synth, e.orc, e.dev = torch, kvs, synth, orc, torch.device("cuda:0")
    return e


class Cache:
    """A paged cache on the GPU and its oracle twin (numpy), with a pinned
    host tier on each side, that decode tokens are appended to."""

    def __init__(self, env, w, lens0, seed, host_tier=True, max_blocks=None):
        torch, kvs = env.torch, env.kvs
        self.env, self.w = env, w
        self.p = Problem(env, w, seq_lens=lens0, max_blocks=max_blocks or w.nb + 1, extra_pages=2)
        p, L = self.p, self.p.L
        self.rng = np.random.default_rng(seed)
        self.fp8 = w.kv_dtype == "e4m3"
        # the state before the first append: summaries of lens0 tokens
        self.summ = p.gpu_summaries()
        self.o_summ = p.or_summaries()
        self.o = {n: (None if p.h[n] is None else p.h[n].copy()) for n in ("k_pool", "v_pool", "k_scales", "v_scales")}
        self.host = {}
        self.o_host = {}
        if host_tier:
            units = L.num_seqs * L.num_kv_heads
            tile = L.block_size * L.head_dim
            shape = (units * L.max_blocks * tile,)
            dt = kvs._TORCH_OF[L.kv_dtype]
            fill = {torch.float32: 3.5, torch.bfloat16: -2.25, torch.uint8: 0x55}[dt]
            for n in ("host_k", "host_v"):
                self.host[n] = torch.full(shape, fill, dtype=dt).pin_memory()
                self.o_host[n] = np_pool(self.host[n]).copy()
            if self.fp8:
                for n in ("host_k_scales", "host_v_scales"):
                    self.host[n] = torch.full((shape[0] // L.quant_group,), -1.0).pin_memory()
                    self.o_host[n] = self.host[n].numpy().copy()
        self.lens = np.asarray(lens0, np.int64)

    def new_token(self):
        """k_new, v_new (+ scales) as stored elements: device tensors and numpy."""
        torch, L = self.env.torch, self.p.L
        out = {}
        for n in ("k", "v"):
            x = torch.from_numpy(self.rng.standard_normal((L.num_seqs, L.num_kv_heads, L.head_dim)).astype(np.float32))
            if self.fp8:
                codes, scales = self.env.synth.quantize_e4m3(x, L.quant_group)
                out[n] = codes
                out[n + "_s"] = scales
            else:
                out[n] = x.to(self.env.kvs._TORCH_OF[L.kv_dtype])
                out[n + "_s"] = None
        return out

    def args(self, tok):
        kvs, dev, inp = self.env.kvs, self.env.dev, self.p.inp
        return kvs.AppendArgs(
            k_new=tok["k"].to(dev), v_new=tok["v"].to(dev),
            k_new_scales=None if tok["k_s"] is None else tok["k_s"].to(dev),
            v_new_scales=None if tok["v_s"] is None else tok["v_s"].to(dev),
            block_table=inp["block_table"], k_pool=inp["k_pool"], v_pool=inp["v_pool"],
            k_scales=inp["k_scales"], v_scales=inp["v_scales"],
            host_k=self.host.get("host_k"), host_v=self.host.get("host_v"),
            host_k_scales=self.host.get("host_k_scales"), host_v_scales=self.host.get("host_v_scales"))

    def oracle_append(self, tok, lens):
        o, h = self.o, self.o_host
        self.env.orc.append_token(
            self.p.OL, np_pool(tok["k"]), np_pool(tok["v"]),
            None if tok["k_s"] is None else tok["k_s"].numpy(),
            None if tok["v_s"] is None else tok["v_s"].numpy(),
            self.p.h["table"], lens, o["k_pool"], o["v_pool"], o["k_scales"], o["v_scales"],
            self.o_summ, h.get("host_k"), h.get("host_v"), h.get("host_k_scales"), h.get("host_v_scales"))

    def set_lens(self, lens):
        self.lens = np.asarray(lens, np.int64)
        self.p.inp["seq_lens"].copy_(self.env.torch.as_tensor(self.lens, dtype=self.env.torch.int32))
        self.p.h["lens"] = self.lens.astype(np.int32)
        self.p.nbs = [(int(n) + self.w.S - 1) // self.w.S for n in self.lens]

    def check(self, what):
        p = self.p
        for n in ("k_pool", "v_pool", "k_scales", "v_scales"):
            if self.o[n] is None:
                continue
            g = np_pool(p.inp[n]) if n.endswith("pool") else p.inp[n].cpu().numpy()
            assert np.array_equal(g.view(np.uint8), self.o[n].view(np.uint8)), f"{what}: {n} differs"
        g = self.summ.double().cpu().numpy()
        for b, n in enumerate(self.lens):
            nb = (int(n) + self.w.S - 1) // self.w.S
            assert np.array_equal(g[b, :, :nb], self.o_summ[b, :, :nb]), f"{what}: summaries of sequence {b} differ"
        for n, t in self.host.items():
            gh = np_pool(t) if n in ("host_k", "host_v") else t.numpy()
            assert np.array_equal(gh.view(np.uint8), self.o_host[n].view(np.uint8)), f"{what}: {n} differs"


APPEND_CASES = [
    # (name, workload, overrides, first lengths, steps)
    ("bf16-s64-d128", "llama8b", {"B": 4, "L": 64 * 6, "layers": 1, "heavy": "none"}, [64 * 3 - 5, 64, 1, 0], 70),
    ("bf16-s16-d64", "llama8b", {"B": 3, "L": 16 * 12, "S": 16, "D": 64, "Hq": 8, "Hkv": 2, "layers": 1,
                                 "heavy": "none"}, [30, 16, 3], 40),
    ("f32-s16", "tiny", {"B": 3, "L": 16 * 10}, [50, 15, 1], 36),
    ("fp8-s64-qg32", "longfp8", {"B": 2, "L": 64 * 5}, [64 * 2 - 3, 64], 67),
    ("fp8-s32-d64-qg16", "longfp8", {"B": 2, "L": 32 * 6, "S": 32, "D": 64, "quant_group": 16}, [40, 32], 35),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_token_steps_match_oracle(env, case):
    name, base, over, lens0, steps = case
    w = env.synth.scaled(env.synth.WORKLOADS[base], **over, k=4)
    print(f"[append {name}] B={w.B} Hkv={w.Hkv} D={w.D} S={w.S} lens0={lens0} steps={steps} {w.kv_dtype}",
          flush=True)
    c = Cache(env, w, lens0, seed=7)
    kvs = env.kvs
    lens = np.asarray(lens0, np.int64)
    for step in range(steps):
        # a sequence that started empty stays empty (nothing is appended to it)
        lens = np.where(np.asarray(lens0) > 0, lens + 1, 0)
        c.set_lens(lens)
        tok = c.new_token()
        kvs.kvs_append_token(c.p.L, c.args(tok), c.p.inp["seq_lens"], c.summ)
        c.oracle_append(tok, lens.astype(np.int32))
        if step % 17 == 16 or step == steps - 1:
            no_device_errors(env)
            c.check(f"step {step}")
    sealed = sum(int(n) // w.S - int(m) // w.S for n, m in zip(lens, lens0))
    print(f"[append {name}] {steps} steps, {sealed} blocks sealed into the host tier")
    assert sealed > 0


FUSED_CASES = [
    # (name, workload, overrides, first lengths, steps, k); k 2 gives one split
    ("bf16-s64-d128", "llama8b", {"B": 3, "L": 64 * 8, "layers": 1}, [64 * 3 - 5, 64 * 5 + 3, 1], 70, 6),
    ("bf16-s64-one-split", "llama8b", {"B": 2, "L": 64 * 6, "layers": 1}, [64 * 2 - 2, 64 + 40], 68, 2),
    ("bf16-s32-d64", "llama8b", {"B": 2, "L": 32 * 10, "S": 32, "D": 64, "Hq": 16, "layers": 1}, [40, 32 * 3], 36,
     5),
    ("fp8-two-launches", "longfp8", {"B": 2, "L": 64 * 5}, [64 * 2 - 3, 64], 67, 4),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_append_attn_in_one_call_matches_two_calls_and_oracle(env, case):
    """kvs_append_sparse_decode_attn over many decode steps (blocks filled and
    sealed on the way) against kvs_append_token + kvs_sparse_decode_attn on
    a second copy of the cache: outputs, pools, summaries and host tiers
    bit-identical at every step; and against the oracle (cache bit-exact,
    attention within the bars).  bf16 runs as one launch (the token's tile
    takes its K row and V column from the arguments, the unit's first split
    workgroup writes it after its attention); fp8 takes the two launches."""
    from test_gpu_parity import check_attn
    name, base, over, lens0, steps, k = case
    torch, kvs, orc = env.torch, env.kvs, env.orc
    w = env.synth.scaled(env.synth.WORKLOADS[base], **over, k=k)
    c1 = Cache(env, w, lens0, seed=31)
    c2 = Cache(env, w, lens0, seed=31)
    L = c1.p.L
    print(f"[append+attn {name}] B={w.B} D={w.D} S={w.S} k={k} splits={kvs.kvs_attn_num_splits(L, k)} "
          f"steps={steps} {w.kv_dtype}", flush=True)
    ws1 = torch.zeros(kvs.kvs_attn_workspace_size(L, k), dtype=torch.uint8, device=env.dev)
    ws2 = torch.zeros_like(ws1)
    lens = np.asarray(lens0, np.int64)
    worst = 0.0
    for step in range(steps):
        lens = lens + 1
        c1.set_lens(lens)
        c2.set_lens(lens)
        tok = c1.new_token()
        c2.new_token()  # keeps the two generators in step
        sel_np = env.synth.random_selection(w, lens, k, seed=step)
        sel = torch.from_numpy(sel_np).to(env.dev)
        o1 = torch.full((L.num_seqs, L.num_q_heads, L.head_dim), float("nan"), device=env.dev)
        o2 = torch.full_like(o1, float("nan"))
        p1, p2 = c1.p, c2.p
        kvs.kvs_append_sparse_decode_attn(L, c1.args(tok), c1.summ, p1.inp["q"], p1.inp["seq_lens"], sel, k,
                                          p1.sm_scale, o1, ws1)
        kvs.kvs_append_token(L, c2.args(tok), p2.inp["seq_lens"], c2.summ)
        kvs.kvs_sparse_decode_attn(L, kvs.KVS_TABLE_PAGED, p2.inp["q"], p2.inp["k_pool"], p2.inp["v_pool"],
                                   p2.inp["k_scales"], p2.inp["v_scales"], p2.inp["block_table"],
                                   p2.inp["seq_lens"], sel, k, p2.sm_scale, o2, ws2)
        torch.cuda.synchronize()
        no_device_errors(env)
        def same(x, y):  # bit for bit (unbuilt summaries hold NaN)
            return torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))
        assert same(o1, o2), f"step {step}: outputs differ"
        for n in ("k_pool", "v_pool", "k_scales", "v_scales"):
            if p1.inp[n] is not None:
                assert same(p1.inp[n], p2.inp[n]), f"step {step}: {n} differs"
        assert same(c1.summ, c2.summ), f"step {step}: summaries differ"
        for n in c1.host:
            assert same(c1.host[n], c2.host[n]), f"step {step}: {n} differs"
        c1.oracle_append(tok, lens.astype(np.int32))
        if step % 11 == 10 or step == steps - 1:
            c1.check(f"step {step}")
            o_out = orc.sparse_attn(p1.OL, p1.inp["q"].double().cpu().numpy(), c1.o["k_pool"], c1.o["v_pool"],
                                    c1.o["k_scales"], c1.o["v_scales"], p1.h["table"], p1.h["lens"], sel_np,
                                    p1.sm_scale)
            err, _ = check_attn(o1, o_out)
            worst = max(worst, err)
    sealed = sum(int(n) // w.S - int(m) // w.S for n, m in zip(lens, lens0))
    print(f"[append+attn {name}] {steps} steps, {sealed} blocks sealed, attention max|err| {worst:.2e}")
    assert sealed > 0


def _drift_q(env, q, rng):
    """Next step's query: a bf16 random walk that keeps most of the last one."""
    torch = env.torch
    x = q.float().cpu().numpy()
    x = 0.8 * x + 0.6 * rng.standard_normal(x.shape)
    return torch.from_numpy(x.astype(np.float32)).to(q.dtype).to(q.device)


SELECT_CASES = [
    # (name, workload, overrides, lens, max_blocks (None: fitted), k, recent, ema, bounds)
    ("window8", "llama8b", {"B": 3, "L": 64 * 90, "layers": 1}, [64 * 90, 64 * 70 + 9, 64 * 10], None, 24, 8,
     False, True),
    ("window8-no-bounds", "llama8b", {"B": 3, "L": 64 * 90, "layers": 1}, [64 * 90, 64 * 70 + 9, 64 * 10], None,
     24, 8, False, False),
    ("ema", "llama8b", {"B": 3, "L": 64 * 90, "layers": 1}, [64 * 90, 64 * 70 + 9, 64 * 10], None, 24, 1, True,
     True),
    ("ema-window16-no-bounds", "llama8b", {"B": 3, "L": 64 * 90, "layers": 1}, [64 * 90, 64 * 33, 64 * 20 + 1],
     None, 20, 16, True, False),
    ("ema-fp8", "longfp8", {"B": 2, "L": 64 * 60}, [64 * 60, 64 * 41 + 3], None, 12, 4, True, True),
    ("ema-f32-s16", "tiny", {"B": 2, "L": 1000}, [1000, 517], None, 10, 3, True, False),
    ("window-matrix-core", "llama8b", {"B": 8, "L": 64 * 300, "layers": 1},
     [64 * 300, 64 * 300 - 7, 64 * 120, 64 * 41 + 5, 64 * 300, 64 * 2, 64 * 40, 64 * 299 + 1], 2048, 40, 8,
     False, False),
]


@pytest.mark.parametrize("case", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_select_ex_window_and_smoothing_over_steps(env, case):
    name, base, over, lens, mb, k, recent, ema, with_bounds = case
    torch, kvs, orc = env.torch, env.kvs, env.orc
    w = env.synth.scaled(env.synth.WORKLOADS[base], **over, k=k)
    p = Problem(env, w, seq_lens=lens, max_blocks=mb if mb else w.nb + 2, extra_pages=3)
    L = p.L
    print(f"[select-ex {name}] units {L.num_seqs * L.num_kv_heads} max_blocks {L.max_blocks} k={k} "
          f"recent={recent} ema={ema} bounds={with_bounds}", flush=True)
    summ = p.gpu_summaries()
    o_summ = p.or_summaries()
    state = torch.full((L.num_seqs, L.num_kv_heads, L.max_blocks), float("nan"), dtype=torch.float64,
                       device=env.dev)
    o_state = np.full(tuple(state.shape), np.nan)
    opts = kvs.SelectOpts(recent_blocks=recent, use_ema=ema, ema_alpha=0.7, ema_state=state if ema else None)
    ws = torch.empty(kvs.kvs_select_workspace_size(L, k), dtype=torch.uint8, device=env.dev)
    rng = np.random.default_rng(99)
    changed = 0
    prev = None
    for step in range(6):
        sel = torch.full((L.num_seqs, L.num_kv_heads, k), -7, dtype=torch.int32, device=env.dev)
        W = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64,
                        device=env.dev) if with_bounds else None
        kvs.kvs_select_topk_ex(L, p.inp["q"], summ, p.inp["seq_lens"], k, opts, None, sel, W, ws)
        no_device_errors(env)
        p.h["q"] = p.inp["q"].double().cpu().numpy()
        o_W = orc.bounds(p.OL, p.h["q"], o_summ, p.h["lens"])
        rank = orc.ema_scores(p.OL, o_W, p.h["lens"], 0.7, o_state) if ema else o_W
        o_sel = orc.select_window(p.OL, rank, p.h["lens"], k, recent)
        if with_bounds:
            gW = W.cpu().numpy()
            for b, nb in enumerate(p.nbs):
                assert np.array_equal(gW[b, :, :nb], o_W[b, :, :nb]), f"step {step}: bounds differ"
        assert np.array_equal(sel.cpu().numpy(), o_sel), f"step {step}: selection differs"
        if ema:
            gs = state.cpu().numpy()
            assert np.array_equal(np.isnan(gs), np.isnan(o_state)), f"step {step}: state NaN pattern differs"
            assert np.array_equal(np.nan_to_num(gs), np.nan_to_num(o_state)), f"step {step}: state differs"
        if prev is not None:
            changed += int((o_sel != prev).any(axis=-1).sum())
        prev = o_sel
        p.inp["q"] = _drift_q(env, p.inp["q"], rng)
    print(f"[select-ex {name}] 6 steps; units whose selection changed between steps: {changed}")


FUSED_CASES = [
    # (name, workload, overrides, lens0, max_blocks, k, recent, ema, bounds)
    ("bf16-fused", "llama8b", {"B": 3, "L": 64 * 40, "layers": 1, "heavy": "none"}, [64 * 30 - 1, 64 * 7, 5],
     None, 12, 2, False, False),
    ("bf16-matrix-core-fused", "llama8b", {"B": 8, "L": 64 * 300, "layers": 1, "heavy": "none"},
     [64 * 290 - 1, 64 * 200, 64 * 100 + 3, 64 * 41 + 5, 64 * 280, 64 * 2, 64 * 40, 64 * 250 + 1], 2048, 40, 4,
     False, False),
    ("bf16-bounds", "llama8b", {"B": 3, "L": 64 * 40, "layers": 1, "heavy": "none"}, [64 * 30 - 1, 64 * 7, 5],
     None, 12, 1, False, True),
    ("bf16-ema", "llama8b", {"B": 3, "L": 64 * 40, "layers": 1, "heavy": "none"}, [64 * 30 - 1, 64 * 7, 5],
     None, 12, 3, True, False),
    ("fp8-fused", "longfp8", {"B": 2, "L": 64 * 40}, [64 * 30 - 1, 64 * 7], None, 10, 2, False, False),
    ("f32-fused", "tiny", {"B": 2, "L": 16 * 40}, [16 * 30 - 1, 16 * 7], None, 10, 2, False, False),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_select_ex_with_token_append(env, case):
    """kvs_select_topk_ex with the append: the cache, summaries and host tier
    come out as the oracle's append leaves them, and the selection is the
    oracle's on the updated summaries -- whether the append runs inside the
    scoring launch or before it."""
    name, base, over, lens0, mb, k, recent, ema, with_bounds = case
    torch, kvs, orc = env.torch, env.kvs, env.orc
    w = env.synth.scaled(env.synth.WORKLOADS[base], **over, k=k)
    c = Cache(env, w, lens0, seed=3, max_blocks=mb)
    p, L = c.p, c.p.L
    print(f"[select-ex+append {name}] units {L.num_seqs * L.num_kv_heads} k={k} recent={recent} ema={ema} "
          f"bounds={with_bounds}", flush=True)
    state = torch.full((L.num_seqs, L.num_kv_heads, L.max_blocks), float("nan"), dtype=torch.float64,
                       device=env.dev)
    o_state = np.full(tuple(state.shape), np.nan)
    opts = kvs.SelectOpts(recent_blocks=recent, use_ema=ema, ema_alpha=0.7, ema_state=state if ema else None)
    ws = torch.empty(kvs.kvs_select_workspace_size(L, k), dtype=torch.uint8, device=env.dev)
    lens = np.asarray(lens0, np.int64)
    for step in range(3):
        lens = lens + 1
        c.set_lens(lens)
        tok = c.new_token()
        sel = torch.full((L.num_seqs, L.num_kv_heads, k), -7, dtype=torch.int32, device=env.dev)
        W = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64,
                        device=env.dev) if with_bounds else None
        kvs.kvs_select_topk_ex(L, p.inp["q"], c.summ, p.inp["seq_lens"], k, opts, c.args(tok), sel, W, ws)
        no_device_errors(env)
        c.oracle_append(tok, lens.astype(np.int32))
        c.check(f"step {step}")
        o_W = orc.bounds(p.OL, p.h["q"], c.o_summ, p.h["lens"])
        rank = orc.ema_scores(p.OL, o_W, p.h["lens"], 0.7, o_state) if ema else o_W
        o_sel = orc.select_window(p.OL, rank, p.h["lens"], k, recent)
        assert np.array_equal(sel.cpu().numpy(), o_sel), f"step {step}: selection differs"
        if with_bounds:
            gW = W.cpu().numpy()
            for b, nb in enumerate(p.nbs):
                assert np.array_equal(gW[b, :, :nb], o_W[b, :, :nb]), f"step {step}: bounds differ"
        if ema:
            assert np.array_equal(np.nan_to_num(state.cpu().numpy()), np.nan_to_num(o_state))


SPLIT_CASES = [
    # (name, workload, overrides, lens0, max_blocks, k, recent, ema)
    ("bf16-self", "llama8b", {"B": 3, "L": 64 * 60, "layers": 1}, [64 * 50 - 1, 64 * 20 + 7, 5], None, 24, 1, False),
    ("bf16-self-window8", "llama8b", {"B": 3, "L": 64 * 60, "layers": 1}, [64 * 50 - 1, 64 * 20 + 7, 64 * 9],
     None, 24, 8, False),
    ("bf16-self-ema", "llama8b", {"B": 2, "L": 64 * 60, "layers": 1}, [64 * 50 - 1, 64 * 33], None, 16, 2, True),
    ("bf16-s32-d64-self", "llama8b", {"B": 2, "L": 32 * 70, "S": 32, "D": 64, "Hq": 16, "layers": 1},
     [32 * 60 + 3, 32 * 11], None, 20, 1, False),
    ("bf16-self-one-split", "llama8b", {"B": 2, "L": 64 * 40, "layers": 1}, [64 * 30, 64 * 4], None, 4, 1, False),
    ("fp8-self", "longfp8", {"B": 2, "L": 64 * 80}, [64 * 70 + 1, 64 * 12], None, 16, 3, False),
    ("bf16-s16-fallback", "llama8b", {"B": 2, "L": 16 * 90, "S": 16, "Hq": 32, "Hkv": 2, "layers": 1},
     [16 * 80 + 5, 16 * 7], None, 20, 2, False),
    ("f32-fallback", "tiny", {"B": 2, "L": 16 * 60}, [16 * 50, 16 * 9 + 2], None, 10, 1, True),
    ("bf16-mb-over-2048-fallback", "llama8b", {"B": 1, "L": 64 * 100, "layers": 1}, [64 * 90 + 3], 2100, 12, 2,
     False),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_score_blocks_then_select_attn(env, case):
    """kvs_score_blocks (with the token append) then kvs_select_attn: the
    scores, the smoothing state and the selection equal the oracle's bit for
    bit (the same selection kvs_select_topk_ex makes), and the attention is
    within the bars, over three decode steps."""
    from test_gpu_parity import check_attn
    name, base, over, lens0, mb, k, recent, ema = case
    torch, kvs, orc = env.torch, env.kvs, env.orc
    w = env.synth.scaled(env.synth.WORKLOADS[base], **over, k=k)
    c = Cache(env, w, lens0, seed=11, max_blocks=mb)
    p, L = c.p, c.p.L
    print(f"[score+select-attn {name}] units {L.num_seqs * L.num_kv_heads} max_blocks {L.max_blocks} k={k} "
          f"recent={recent} ema={ema} splits={kvs.kvs_attn_num_splits(L, k)}", flush=True)
    state = torch.full((L.num_seqs, L.num_kv_heads, L.max_blocks), float("nan"), dtype=torch.float64,
                       device=env.dev)
    o_state = np.full(tuple(state.shape), np.nan)
    opts = kvs.SelectOpts(recent_blocks=recent, use_ema=ema, ema_alpha=0.7, ema_state=state if ema else None)
    scores = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64, device=env.dev)
    aws = torch.zeros(kvs.kvs_attn_workspace_size(L, k), dtype=torch.uint8, device=env.dev)
    sws = torch.empty(kvs.kvs_select_workspace_size(L, k), dtype=torch.uint8, device=env.dev)
    lens = np.asarray(lens0, np.int64)
    rng = np.random.default_rng(5)
    for step in range(3):
        lens = lens + 1
        c.set_lens(lens)
        tok = c.new_token()
        sel = torch.full((L.num_seqs, L.num_kv_heads, k), -7, dtype=torch.int32, device=env.dev)
        out = torch.full((L.num_seqs, L.num_q_heads, L.head_dim), float("nan"), device=env.dev)
        kvs.kvs_score_blocks(L, p.inp["q"], c.summ, p.inp["seq_lens"], opts, c.args(tok), scores, None)
        kvs.kvs_select_attn(L, p.inp["q"], p.inp["k_pool"], p.inp["v_pool"], p.inp["k_scales"], p.inp["v_scales"],
                            p.inp["block_table"], p.inp["seq_lens"], scores, k, recent, sel, p.sm_scale, out, aws)
        no_device_errors(env)
        c.oracle_append(tok, lens.astype(np.int32))
        c.check(f"step {step}")
        p.h["q"] = p.inp["q"].double().cpu().numpy()
        o_W = orc.bounds(p.OL, p.h["q"], c.o_summ, p.h["lens"])
        rank = orc.ema_scores(p.OL, o_W, p.h["lens"], 0.7, o_state) if ema else o_W
        gs = scores.cpu().numpy()
        for b, nb in enumerate(p.nbs):
            # fused append (no smoothing): the newest block's score is unspecified
            upto = nb if ema else nb - 1
            assert np.array_equal(gs[b, :, :upto], rank[b, :, :upto]), f"step {step}: scores differ"
            assert np.isneginf(gs[b, :, nb:]).all()
        o_sel = orc.select_window(p.OL, rank, p.h["lens"], k, recent)
        assert np.array_equal(sel.cpu().numpy(), o_sel), f"step {step}: selection differs"
        # the separate selection launch picks the same blocks from the same scores
        if not ema:
            sel2 = torch.full_like(sel, -7)
            kvs.kvs_select_topk_ex(L, p.inp["q"], c.summ, p.inp["seq_lens"], k,
                                   kvs.SelectOpts(recent_blocks=recent), None, sel2, None, sws)
            no_device_errors(env)
            assert torch.equal(sel, sel2), f"step {step}: kvs_select_topk_ex picks other blocks"
        o_out = orc.sparse_attn(p.OL, p.h["q"], c.o["k_pool"], c.o["v_pool"], c.o["k_scales"], c.o["v_scales"],
                                p.h["table"], p.h["lens"], o_sel, p.sm_scale)
        err, rel = check_attn(out, o_out)
        p.inp["q"] = _drift_q(env, p.inp["q"], rng)
    print(f"[score+select-attn {name}] attention max|err| {err:.2e} rel L2 {rel:.2e}")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_fused_append_error_paths_leave_the_cache_alone(env, kind):
    """kvs_score_blocks with the token append, where sequence 0's length is
    past the table (flagged KVS_DEVERR_SEQLEN) and sequence 1's newest block
    maps to a page past the pool (flagged KVS_DEVERR_TABLE): neither gets the
    token, while sequence 2 is appended (K/V, summary, scales) exactly as the
    oracle appends it and its scores are exact.  Every workgroup issues the
    same token loads whether or not it appends, so this also runs the
    kernel's spare-address path for all of them."""
    torch, kvs, orc = env.torch, env.kvs, env.orc
    base = "llama8b" if kind == "bf16" else "longfp8"
    w = env.synth.scaled(env.synth.WORKLOADS[base], B=3, L=64 * 20, k=8, layers=1)
    c = Cache(env, w, [64 * 20 - 9, 64 * 13 + 7, 64 * 11 + 30], seed=23, host_tier=False)
    p, L = c.p, c.p.L
    lens = c.lens + 1
    c.set_lens(lens)
    bad_lens = lens.copy()
    bad_lens[0] = L.max_blocks * L.block_size + 5
    p.inp["seq_lens"].copy_(torch.as_tensor(bad_lens, dtype=torch.int32))
    j1 = int(lens[1] - 1) // L.block_size
    tbl = p.inp["block_table"].clone()
    p.inp["block_table"][1, j1] = L.num_pages + 1000
    tok = c.new_token()
    scores = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64, device=env.dev)
    kvs.kvs_score_blocks(L, p.inp["q"], c.summ, p.inp["seq_lens"], kvs.SelectOpts(), c.args(tok), scores, None)
    torch.cuda.synchronize()
    flags = kvs.kvs_device_errors(clear=True)
    assert flags & kvs.KVS_DEVERR_SEQLEN and flags & kvs.KVS_DEVERR_TABLE, f"flags {flags:#x}"
    p.inp["block_table"].copy_(tbl)
    p.inp["seq_lens"].copy_(torch.as_tensor(lens, dtype=torch.int32))
    # the oracle appends to sequence 2 only (a length of 0 appends nothing)
    c.oracle_append(tok, np.asarray([0, 0, lens[2]], np.int32))
    c.check("error paths")
    p.h["q"] = p.inp["q"].double().cpu().numpy()
    o_W = orc.bounds(p.OL, p.h["q"], c.o_summ, p.h["lens"])
    nb2 = p.nbs[2]
    gs = scores.cpu().numpy()
    assert np.array_equal(gs[2, :, :nb2 - 1], o_W[2, :, :nb2 - 1]), "sequence 2's scores differ"
    no_device_errors(env)
    print(f"[fused append errors {kind}] flags {flags:#x}; sequence 2 appended, 0 and 1 untouched")


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_prefetch_pipeline_matches_oracle_and_sequential_hot_steps(env, kind):
    """Layers' swap-ins issued ahead (page-table steps two layers ahead on
    the compute stream, copies one layer ahead on a second stream while
    layer i attends) give exactly the outputs, page tables and slot states of the
    same steps run one after another, and match the oracle: every step's
    miss list and count, the final page tables, owners and stamps bit-exact,
    every step's attention within the bars."""
    torch, kvs, synth = env.torch, env.kvs, env.synth
    from query_aware_sparse_kvs_amd.step import HotBufferStep, HotPrefetchPipeline
    from test_gpu_parity import check_attn
    orc = env.orc
    if kind == "bf16":
        w = synth.scaled(synth.WORKLOADS["llama8b"], B=2, L=64 * 40, Hkv=2, Hq=8, layers=1, k=10)
    else:
        w = synth.scaled(synth.WORKLOADS["longfp8"], B=2, L=64 * 40 - 9, Hkv=2, Hq=8, k=10)
    p = Problem(env, w)
    L = p.L
    n_layers, steps, ns = 3, 7, 12
    units = L.num_seqs * L.num_kv_heads
    print(f"[prefetch {kind}] {n_layers} layers x {steps} steps, units {units}, k {w.k}, slots {ns}", flush=True)
    sel0 = synth.random_selection(w, p.h["lens"], w.k, seed=4)
    stream = synth.drift_selections(sel0, w.nb, n_layers * steps + 2, 3, seed=5)
    sels = torch.from_numpy(stream).to(env.dev)
    pages = p.inp["block_table"].long().cpu()
    host = [None if p.inp[n] is None else p.inp[n].cpu()[pages].transpose(1, 2).contiguous().pin_memory()
            for n in ("k_pool", "v_pool", "k_scales", "v_scales")]
    seq = [HotBufferStep(L, w.k, ns, env.dev) for _ in range(n_layers)]
    pip = [HotBufferStep(L, w.k, ns, env.dev) for _ in range(n_layers)]
    pipe = HotPrefetchPipeline(pip, env.dev)
    outs_seq, outs_pip, miss_pip = [], [], []
    t_of = lambda i: 1 + i  # stream entry of step i (entry 0 is the warm start)
    for h in seq + pip:
        h.run(0, sels[0], p.inp["q"], p.inp["seq_lens"], *host)
    for i in range(n_layers * steps):
        outs_seq.append(seq[i % n_layers].run(t_of(i), sels[t_of(i)], p.inp["q"], p.inp["seq_lens"], *host).clone())
    layer_of = lambda i: i % n_layers
    lookup_args = lambda i: (t_of(i), sels[t_of(i)])
    for i in range(n_layers * steps):
        # lookups two steps ahead, copies one step ahead, then step i's attention
        out = pipe.step(i, layer_of, lookup_args, host, p.inp["q"], sels[t_of(i)], p.inp["seq_lens"])
        outs_pip.append(out.clone())
        # this buffer's next lookup (step i + n_layers) is enqueued later on the same stream
        miss_pip.append((pip[i % n_layers].miss_list.clone(), pip[i % n_layers].miss_count.clone()))
    N = n_layers * steps
    # the pipeline has issued the lookups and copies of the steps after N-1
    # already: take the sequential buffers to the same point
    for m in range(N, pipe.next_lookup):
        seq[layer_of(m)].lookup(*lookup_args(m))
        if m < pipe.next_copy:
            seq[layer_of(m)].copy(*host)
    torch.cuda.synchronize()
    no_device_errors(env)
    for i, (a, b) in enumerate(zip(outs_seq, outs_pip)):
        assert torch.equal(a, b), f"step {i}: outputs differ"
    for a, b in zip(seq, pip):
        for n in ("page_table", "slot_owner", "slot_stamp", "hot_k", "hot_v", "hot_ks", "hot_vs"):
            if getattr(a, n) is not None:
                assert torch.equal(getattr(a, n), getattr(b, n)), f"{n} differs"
    # the oracle: each buffer's LRU state stepped through its selections
    pt = np.full((n_layers, units, w.nb), -1, np.int32)
    owner = np.full((n_layers, units, ns), -1, np.int32)
    stamp = np.full((n_layers, units, ns), -1, np.int64)
    for l in range(n_layers):
        for u in range(units):
            orc.hot_step(w.nb, ns, 0, u * ns, stream[0].reshape(units, -1)[u], pt[l, u], owner[l, u], stamp[l, u])
    worst = 0.0
    for i in range(n_layers * steps):
        l, t = i % n_layers, t_of(i)
        ml, mc = [], []
        for u in range(units):
            m, c = orc.hot_step(w.nb, ns, t, u * ns, stream[t].reshape(units, -1)[u], pt[l, u], owner[l, u],
                                stamp[l, u])
            ml.append(m)
            mc.append(c)
        g_ml, g_mc = miss_pip[i]
        assert np.array_equal(g_ml.cpu().numpy().reshape(units, -1), np.stack(ml)), f"step {i}: miss lists"
        assert np.array_equal(g_mc.cpu().numpy().reshape(-1), np.array(mc)), f"step {i}: miss counts"
        err, _ = check_attn(outs_pip[i], p.or_attn(stream[t]))
        worst = max(worst, err)
    for m in range(N, pipe.next_lookup):  # the lookups issued ahead
        for u in range(units):
            orc.hot_step(w.nb, ns, t_of(m), u * ns, stream[t_of(m)].reshape(units, -1)[u], pt[layer_of(m), u],
                         owner[layer_of(m), u], stamp[layer_of(m), u])
    for l in range(n_layers):
        assert np.array_equal(pip[l].page_table.cpu().numpy().reshape(units, -1), pt[l])
        assert np.array_equal(pip[l].slot_owner.cpu().numpy().reshape(units, -1), owner[l])
        assert np.array_equal(pip[l].slot_stamp.cpu().numpy().reshape(units, -1), stamp[l])
    print(f"[prefetch {kind}] pipelined = sequential; tables and miss lists = oracle; max|err| {worst:.2e}")


MEAN_CASES = [
    # (name, workload, overrides, lens0, k, recent, append, bounds)
    ("bf16-bounds", "llama8b", {"B": 3, "L": 64 * 40, "layers": 1}, [64 * 30 - 1, 64 * 7, 5], 12, 1, False, True),
    ("bf16-append-window", "llama8b", {"B": 3, "L": 64 * 40, "layers": 1}, [64 * 30 - 1, 64 * 7 + 63, 5], 12, 3,
     True, False),
    ("bf16-s32-d64-g4-append", "llama8b", {"B": 2, "L": 32 * 50, "S": 32, "D": 64, "Hq": 16, "layers": 1},
     [32 * 40 + 3, 32 * 11 - 1], 10, 2, True, True),
    ("fp8-append", "longfp8", {"B": 2, "L": 64 * 40}, [64 * 30 - 1, 64 * 7], 10, 2, True, False),
    ("f32-s16-append", "tiny", {"B": 2, "L": 16 * 40}, [16 * 30 - 1, 16 * 7], 10, 1, True, True),
]


@pytest.mark.parametrize("case", MEAN_CASES, ids=[c[0] for c in MEAN_CASES])
def test_mean_summaries_scores_and_selection(env, case):
    """Mean summaries (kvs_build_summaries_ex), blocks ranked by q.mean
    (kvs_select_topk_ex and kvs_score_blocks + kvs_select_attn with
    summary_kind = mean), with and without the token append: the mean table,
    the scores and the selections equal the oracle's bit for bit, the
    attention is within the bars."""
    from test_gpu_parity import check_attn
    name, base, over, lens0, k, recent, with_append, with_bounds = case
    torch, kvs, orc = env.torch, env.kvs, env.orc
    w = env.synth.scaled(env.synth.WORKLOADS[base], **over, k=k)
    c = Cache(env, w, lens0, seed=21)
    p, L = c.p, c.p.L
    print(f"[mean {name}] units {L.num_seqs * L.num_kv_heads} max_blocks {L.max_blocks} k={k} recent={recent} "
          f"append={with_append} bounds={with_bounds}", flush=True)
    mean = torch.full((L.num_seqs, L.num_kv_heads, L.max_blocks, L.head_dim), float("nan"), device=env.dev)
    kvs.kvs_build_summaries_ex(L, kvs.KVS_SUMM_MEAN, p.inp["k_pool"], p.inp["k_scales"], p.inp["block_table"],
                               p.inp["seq_lens"], None, L.max_blocks, mean)
    no_device_errors(env)
    opts = kvs.SelectOpts(recent_blocks=recent, summary_kind=kvs.KVS_SUMM_MEAN)
    sws = torch.empty(kvs.kvs_select_workspace_size(L, k), dtype=torch.uint8, device=env.dev)
    aws = torch.zeros(kvs.kvs_attn_workspace_size(L, k), dtype=torch.uint8, device=env.dev)
    scores = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64, device=env.dev)
    lens = np.asarray(lens0, np.int64)
    for step in range(3):
        tok = None
        if with_append:
            lens = lens + 1
            c.set_lens(lens)
            tok = c.new_token()
        o_mean = orc.summaries_mean(p.OL, c.o["k_pool"] if with_append else p.h["k_pool"],
                                    c.o["k_scales"] if with_append else p.h["k_scales"], p.h["table"], p.h["lens"])
        sel = torch.full((L.num_seqs, L.num_kv_heads, k), -7, dtype=torch.int32, device=env.dev)
        W = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64,
                        device=env.dev) if with_bounds else None
        kvs.kvs_select_topk_ex(L, p.inp["q"], mean, p.inp["seq_lens"], k, opts,
                               c.args(tok) if tok is not None else None, sel, W, sws)
        no_device_errors(env)
        if tok is not None:
            c.oracle_append(tok, lens.astype(np.int32))
            o_mean = orc.summaries_mean(p.OL, c.o["k_pool"], c.o["k_scales"], p.h["table"], p.h["lens"])
            for n in ("k_pool", "v_pool"):
                assert np.array_equal(np_pool(p.inp[n]).view(np.uint8), c.o[n].view(np.uint8)), f"{n} differs"
        gm = mean.cpu().numpy()
        for b, nb in enumerate(p.nbs):
            assert np.array_equal(gm[b, :, :nb], o_mean[b, :, :nb]), f"step {step}: mean table differs"
        o_W = orc.mean_scores(p.OL, p.h["q"], o_mean, p.h["lens"])
        if with_bounds:
            gW = W.cpu().numpy()
            for b, nb in enumerate(p.nbs):
                assert np.array_equal(gW[b, :, :nb], o_W[b, :, :nb]), f"step {step}: mean scores differ"
        o_sel = orc.select_window(p.OL, o_W, p.h["lens"], k, recent)
        assert np.array_equal(sel.cpu().numpy(), o_sel), f"step {step}: selection differs"
        # the same scores and selection through kvs_score_blocks + kvs_select_attn
        kvs.kvs_score_blocks(L, p.inp["q"], mean, p.inp["seq_lens"], opts, None, scores, None)
        out = torch.full((L.num_seqs, L.num_q_heads, L.head_dim), float("nan"), device=env.dev)
        sel2 = torch.full_like(sel, -7)
        kvs.kvs_select_attn(L, p.inp["q"], p.inp["k_pool"], p.inp["v_pool"], p.inp["k_scales"], p.inp["v_scales"],
                            p.inp["block_table"], p.inp["seq_lens"], scores, k, recent, sel2, p.sm_scale, out, aws)
        no_device_errors(env)
        gs = scores.cpu().numpy()
        for b, nb in enumerate(p.nbs):
            assert np.array_equal(gs[b, :, :nb], o_W[b, :, :nb]), f"step {step}: kvs_score_blocks differs"
        assert torch.equal(sel2, sel), f"step {step}: kvs_select_attn picks other blocks"
        pools = c.o if with_append else p.h
        o_out = orc.sparse_attn(p.OL, p.h["q"], pools["k_pool"], pools["v_pool"], pools["k_scales"],
                                pools["v_scales"], p.h["table"], p.h["lens"], o_sel, p.sm_scale)
        err, rel = check_attn(out, o_out)
    print(f"[mean {name}] attention max|err| {err:.2e} rel L2 {rel:.2e}")


@pytest.mark.parametrize("base,over", [("llama8b", {"B": 5, "L": 64 * 20, "layers": 1}),
                                       ("longfp8", {"B": 5, "L": 64 * 20})],
                         ids=["bf16", "fp8"])
def test_select_attn_empty_short_and_all_block_sequences(env, base, over):
    """kvs_select_attn on ragged lengths: an empty sequence (no blocks: all
    -1, a zero output row), a one-token and a one-block sequence, one whose
    blocks all fit in k, and a long one; selections equal the oracle's and
    attention is within the bars."""
    from test_gpu_parity import check_attn
    torch, kvs, orc = env.torch, env.kvs, env.orc
    k = 6
    lens = [0, 1, 64, 64 * 5 + 7, 64 * 20]
    w = env.synth.scaled(env.synth.WORKLOADS[base], **over, k=k)
    p = Problem(env, w, seq_lens=lens, max_blocks=w.nb + 1, extra_pages=2)
    L = p.L
    print(f"[edge {base}] lens {lens} k={k} splits={kvs.kvs_attn_num_splits(L, k)}", flush=True)
    summ = p.gpu_summaries()
    scores = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64, device=env.dev)
    kvs.kvs_score_blocks(L, p.inp["q"], summ, p.inp["seq_lens"], None, None, scores, None)
    sel = torch.full((L.num_seqs, L.num_kv_heads, k), -7, dtype=torch.int32, device=env.dev)
    out = torch.full((L.num_seqs, L.num_q_heads, L.head_dim), float("nan"), device=env.dev)
    aws = torch.zeros(kvs.kvs_attn_workspace_size(L, k), dtype=torch.uint8, device=env.dev)
    kvs.kvs_select_attn(L, p.inp["q"], p.inp["k_pool"], p.inp["v_pool"], p.inp["k_scales"], p.inp["v_scales"],
                        p.inp["block_table"], p.inp["seq_lens"], scores, k, 2, sel, p.sm_scale, out, aws)
    no_device_errors(env)
    o_summ = p.or_summaries()
    W = p.or_bounds(o_summ)
    gs = scores.cpu().numpy()
    for b, nb in enumerate(p.nbs):
        assert np.array_equal(gs[b, :, :nb], W[b, :, :nb])
        assert np.isneginf(gs[b, :, nb:]).all()
    o_sel = orc.select_window(p.OL, W, p.h["lens"], k, 2)
    assert np.array_equal(sel.cpu().numpy(), o_sel)
    assert (sel[0] == -1).all() and (out[0] == 0).all()
    check_attn(out, p.or_attn(o_sel))


HOT_APPEND_CASES = [
    # (name, workload, overrides, first lengths, steps, k, hot slots per unit)
    ("bf16-s16-d64", "llama8b", {"B": 2, "L": 16 * 12, "S": 16, "D": 64, "Hq": 8, "Hkv": 2, "layers": 1,
                                 "heavy": "none"}, [16 * 4 - 3, 16 * 2 + 5], 36, 5, 7),
    ("fp8-s32-qg32", "longfp8", {"B": 2, "L": 32 * 8, "S": 32}, [32 * 3 - 2, 40], 40, 4, 6),
]


@pytest.mark.parametrize("case", HOT_APPEND_CASES, ids=[c[0] for c in HOT_APPEND_CASES])
def test_hot_buffer_decode_loop_with_appends(env, case):
    """A decode loop over the hot buffer (page "KV 稀疏化", §7) that appends a
    token every step, across block boundaries: kvs_append_token (full blocks
    sealed to the host tier), the selection on the updated summaries, the
    swap-in with the paged cache as the live source of each sequence's
    newest block, and the attention through the hot table.  Every step
    against the oracle: pools, host tier and summaries, the selection, page
    table, owners, stamps, miss lists and counts bit-exact; every resident
    slot byte-equal to its block in the host tier, the newest block's to the
    paged cache; attention within the bars.  Without the live source the
    newest block's slot would miss the tokens appended after its copy."""
    torch, kvs, orc = env.torch, env.kvs, env.orc
    from query_aware_sparse_kvs_amd.step import HotBufferStep
    from test_gpu_parity import check_attn
    name, base, over, lens0, steps, k, ns = case
    w = env.synth.scaled(env.synth.WORKLOADS[base], **over, k=k)
    c = Cache(env, w, lens0, seed=31)
    p, L = c.p, c.p.L
    S, Hkv, MB = L.block_size, L.num_kv_heads, L.max_blocks
    units = L.num_seqs * Hkv
    # the blocks already full before the loop are in the host tier, as their
    # seal would have put them
    table = p.h["table"]
    per_tile = {"k": S * L.head_dim, "s": S * (L.head_dim // L.quant_group) if c.fp8 else 0}
    for b, n in enumerate(lens0):
        for j in range(n // S):
            for g in range(Hkv):
                u, t = b * Hkv + g, table[b, j] * Hkv + g
                for hn, pn, sz in (("host_k", "k_pool", "k"), ("host_v", "v_pool", "k"),
                                   ("host_k_scales", "k_scales", "s"), ("host_v_scales", "v_scales", "s")):
                    if hn not in c.host:
                        continue
                    n_el = per_tile[sz]
                    src_t = p.inp[pn].view(-1)[t * n_el:(t + 1) * n_el].cpu()
                    c.host[hn].view(-1)[(u * MB + j) * n_el:(u * MB + j + 1) * n_el] = src_t
                    c.o_host[hn].reshape(-1)[(u * MB + j) * n_el:(u * MB + j + 1) * n_el] = \
                        c.o[pn].reshape(-1)[t * n_el:(t + 1) * n_el]
    hs = HotBufferStep(L, k, ns, env.dev)
    live = kvs.HotLive(p.inp["k_pool"], p.inp["v_pool"], p.inp["k_scales"], p.inp["v_scales"],
                       p.inp["block_table"], p.inp["seq_lens"])
    pt = np.full((units, MB), -1, np.int32)
    owner = np.full((units, ns), -1, np.int32)
    stamp = np.full((units, ns), -1, np.int64)
    host = [c.host.get(n) for n in ("host_k", "host_v", "host_k_scales", "host_v_scales")]
    print(f"[hot-append {name}] lens {lens0} -> +{steps}, k {k}, slots {ns}", flush=True)
    for t in range(steps):
        tok = c.new_token()
        c.set_lens(c.lens + 1)
        lens = c.lens.astype(np.int32)
        kvs.kvs_append_token(L, c.args(tok), p.inp["seq_lens"], c.summ)
        c.oracle_append(tok, lens)
        c.check(f"step {t}")
        sel, _ = p.gpu_select(c.summ, k, with_bounds=False)
        osel = orc.select(p.OL, orc.bounds(p.OL, p.h["q"], c.o_summ, lens), lens, k)
        assert np.array_equal(sel.cpu().numpy(), osel), f"step {t}: selection differs"
        hs.swap_in(t, sel, *host, live=live)
        misses, counts = [], []
        for u in range(units):
            m, cnt = orc.hot_step(MB, ns, t, u * ns, osel.reshape(units, -1)[u], pt[u], owner[u], stamp[u])
            misses.append(m)
            counts.append(cnt)
        assert np.array_equal(hs.page_table.cpu().numpy().reshape(units, -1), pt), f"step {t}: page table"
        assert np.array_equal(hs.slot_owner.cpu().numpy().reshape(units, -1), owner), f"step {t}: owners"
        assert np.array_equal(hs.slot_stamp.cpu().numpy().reshape(units, -1), stamp), f"step {t}: stamps"
        assert np.array_equal(hs.miss_list.cpu().numpy().reshape(units, -1), np.stack(misses)), f"step {t}"
        assert np.array_equal(hs.miss_count.cpu().numpy().reshape(-1), np.array(counts)), f"step {t}"
        no_device_errors(env)
        # slot contents: the newest block from the paged cache, the others from the host tier
        hot = {"k": hs.hot_k, "v": hs.hot_v, "ks": hs.hot_ks, "vs": hs.hot_vs}
        pools = {"k": p.inp["k_pool"], "v": p.inp["v_pool"], "ks": p.inp["k_scales"], "vs": p.inp["v_scales"]}
        hosts = {"k": host[0], "v": host[1], "ks": host[2], "vs": host[3]}
        for key in ("k", "v", "ks", "vs"):
            if hot[key] is None:
                continue
            n_el = hot[key].numel() // (units * ns)
            hv = hot[key].cpu().reshape(units * ns, n_el)
            pv = pools[key].cpu().reshape(-1, n_el)
            hh = hosts[key].reshape(units * MB, n_el)
            for u in range(units):
                b, g = divmod(u, Hkv)
                newest = (int(lens[b]) - 1) // S
                for s in range(ns):
                    j = int(owner[u, s])
                    if j < 0:
                        continue
                    want = pv[table[b, j] * Hkv + g] if j == newest else hh[u * MB + j]
                    got = hv[u * ns + s]
                    if got.dtype == torch.bfloat16:  # compare bit patterns
                        got, want = got.view(torch.int16), want.view(torch.int16)
                    assert torch.equal(got, want), f"step {t}: slot {s} of unit {u} (block {j}, {key})"
        out = hs.attend(p.inp["q"], sel, p.inp["seq_lens"])
        no_device_errors(env)
        ref = orc.sparse_attn(p.OL, p.h["q"], c.o["k_pool"], c.o["v_pool"], c.o["k_scales"], c.o["v_scales"],
                              table, lens, osel, p.sm_scale)
        check_attn(out, ref)
