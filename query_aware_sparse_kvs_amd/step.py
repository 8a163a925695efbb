"""Decode-step drivers: chain the C entry points of libkvs for one layer and
own the device buffers they need (selection, workspaces, output, hot-buffer
state).  All arithmetic runs in the library's kernels; torch only allocates.
"""
from __future__ import annotations

import math

import torch

from . import kvs


def split_batch(num_seqs: int, parts: int):
    """[b0, b1) ranges of `parts` near-equal slices of the batch (empty ones dropped)."""
    parts = max(1, min(parts, num_seqs)) if num_seqs > 0 else 1
    bounds = [num_seqs * i // parts for i in range(parts + 1)]
    return [(bounds[i], bounds[i + 1]) for i in range(parts) if bounds[i + 1] > bounds[i]] or [(0, 0)]


class SparseDecodeStep:
    """One layer's decode step over a paged KV cache (page "KV 稀疏化", §5
    "Quest"): rebuild the summary of each sequence's newest block (its K row
    was just appended) while scoring and selecting the top-k blocks, then
    attend over them.

    (sequence, KV head) units never interact, so with parts > 1 the batch is
    cut into that many slices of sequences whose calls run as independent
    chains on their own streams (joined back into the caller's stream): one
    slice's selection and short kernels overlap another slice's attention.
    Every slice is the same computation on its rows; results are identical.
    """

    def __init__(self, layout: kvs.Layout, k: int, device="cuda", parts: int = 1):
        L = self.layout = layout
        self.k = k
        dev = torch.device(device)
        self.sel = torch.empty((L.num_seqs, L.num_kv_heads, k), dtype=torch.int32, device=dev)
        self.out = torch.empty((L.num_seqs, L.num_q_heads, L.head_dim), dtype=torch.float32, device=dev)
        self.sm_scale = 1.0 / math.sqrt(L.head_dim)
        self.slices = []
        for b0, b1 in split_batch(L.num_seqs, parts):
            Lp = kvs.Layout(b1 - b0, L.num_q_heads, L.num_kv_heads, L.head_dim, L.block_size, L.max_blocks,
                            L.num_pages, L.q_dtype, L.kv_dtype, L.quant_group)
            sws = torch.empty(max(kvs.kvs_select_workspace_size(Lp, k), 1), dtype=torch.uint8, device=dev)
            aws = torch.zeros(max(kvs.kvs_attn_workspace_size(Lp, k), 1), dtype=torch.uint8, device=dev)
            self.slices.append((b0, b1, Lp, sws, aws))
        self.streams = [torch.cuda.Stream(device=dev) for _ in self.slices[1:]]
        # whole-batch workspaces for the single-chain path
        self.select_ws = torch.empty(max(kvs.kvs_select_workspace_size(L, k), 1), dtype=torch.uint8, device=dev)
        self.scores = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64, device=dev)
        self.attn_ws = torch.zeros(max(kvs.kvs_attn_workspace_size(L, k), 1), dtype=torch.uint8, device=dev)

    def new_summaries(self, device="cuda") -> torch.Tensor:
        L = self.layout
        return torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks, 2, L.head_dim),
                           dtype=L.summary_dtype, device=device)

    def prefill_summaries(self, k_pool, k_scales, block_table, seq_lens, summaries, stream=None):
        kvs.kvs_build_summaries(self.layout, k_pool, k_scales, block_table, seq_lens, None,
                                self.layout.max_blocks, summaries, stream)

    def _chain(self, L, sws, aws, sl, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens,
               summaries, bounds_out, stream):
        k = self.k
        kvs.kvs_select_topk_append(L, q[sl], k_pool, k_scales, block_table[sl], seq_lens[sl], summaries[sl], k,
                                   self.sel[sl], None if bounds_out is None else bounds_out[sl], sws, stream)
        kvs.kvs_sparse_decode_attn(L, kvs.KVS_TABLE_PAGED, q[sl], k_pool, v_pool, k_scales, v_scales,
                                   block_table[sl], seq_lens[sl], self.sel[sl], k, self.sm_scale,
                                   self.out[sl], aws, stream)

    def run_decode(self, q, tok: kvs.AppendArgs, seq_lens, summaries, opts: kvs.SelectOpts | None = None,
                   bounds_out=None, stream=None) -> torch.Tensor:
        """A whole decode layer-step on one chain: the decode token appended
        to the cache (its block's summary updated incrementally; a block that
        fills is sealed into tok's host tier, if any), the blocks scored and
        selected with `opts` (recent window, score smoothing), attention over
        the selection."""
        L, k = self.layout, self.k
        kvs.kvs_select_topk_ex(L, q, summaries, seq_lens, k, opts, tok, self.sel, bounds_out, self.select_ws,
                               stream)
        kvs.kvs_sparse_decode_attn(L, kvs.KVS_TABLE_PAGED, q, tok.k_pool, tok.v_pool, tok.k_scales, tok.v_scales,
                                   tok.block_table, seq_lens, self.sel, k, self.sm_scale, self.out,
                                   self.attn_ws, stream)
        return self.out

    def run_decode_fused(self, q, tok: kvs.AppendArgs, seq_lens, summaries,
                         opts: kvs.SelectOpts | None = None, bounds_out=None, stream=None) -> torch.Tensor:
        """run_decode's layer-step with the top-k done inside the attention
        launch: kvs_score_blocks (append, scores), then kvs_select_attn."""
        L, k = self.layout, self.k
        kvs.kvs_score_blocks(L, q, summaries, seq_lens, opts, tok, self.scores, bounds_out, stream)
        recent = opts.recent_blocks if opts is not None else 1
        kvs.kvs_select_attn(L, q, tok.k_pool, tok.v_pool, tok.k_scales, tok.v_scales, tok.block_table, seq_lens,
                            self.scores, k, recent, self.sel, self.sm_scale, self.out, self.attn_ws, stream)
        return self.out

    def run_decode_best(self, q, tok: kvs.AppendArgs, seq_lens, summaries, stream=None) -> torch.Tensor:
        """The decode layer-step by the cheaper route for this layout: the
        top-k inside the attention launch (run_decode_fused), unless the
        library scores this layout on the matrix cores, where the separate
        selection launch is cheaper (run_decode)."""
        if kvs.kvs_select_uses_matrix_cores(self.layout, self.k):
            return self.run_decode(q, tok, seq_lens, summaries, stream=stream)
        return self.run_decode_fused(q, tok, seq_lens, summaries, stream=stream)

    def run(self, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, summaries,
            bounds_out=None, stream=None) -> torch.Tensor:
        """summaries: in/out, every block but the newest already summarised.
        stream: None (torch's current stream) or a torch.cuda.Stream."""
        args = (q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, summaries, bounds_out)
        if len(self.slices) == 1:
            self._chain(self.layout, self.select_ws, self.attn_ws, slice(None), *args, stream)
            return self.out
        cur = torch.cuda.current_stream() if stream is None else stream
        fork = torch.cuda.Event()
        fork.record(cur)
        joins = []
        for i, (b0, b1, Lp, sws, aws) in enumerate(self.slices):
            s = cur if i == 0 else self.streams[i - 1]
            if i:
                s.wait_event(fork)
            with torch.cuda.stream(s):
                self._chain(Lp, sws, aws, slice(b0, b1), *args, None)
            if i:
                e = torch.cuda.Event()
                e.record(s)
                joins.append(e)
        for e in joins:
            cur.wait_event(e)
        return self.out


class HotBufferStep:
    """One layer's decode step with a hot device buffer over a pinned host
    tier (page "KV 稀疏化", §7 "HiSparse"): page-table lookup, LRU slot
    assignment and swap-in of the missed blocks, then attention through the
    hot page table.  State starts empty (every entry -1).  In a decode loop
    that appends tokens, pass `live` (the paged cache the append writes) to
    the swap-in, after the append: each sequence's newest block, which the
    host tier does not hold until it is sealed, is then copied from there."""

    def __init__(self, layout: kvs.Layout, k: int, num_slots: int, device="cuda"):
        L = layout
        self.k, self.ns = k, num_slots
        dev = torch.device(device)
        units = L.num_seqs * L.num_kv_heads
        self.host_layout = layout
        self.hot_layout = kvs.Layout(L.num_seqs, L.num_q_heads, L.num_kv_heads, L.head_dim,
                                     L.block_size, L.max_blocks, units * num_slots, L.q_dtype,
                                     L.kv_dtype, L.quant_group)
        self.page_table = torch.full((L.num_seqs, L.num_kv_heads, L.max_blocks), -1, dtype=torch.int32, device=dev)
        self.slot_owner = torch.full((L.num_seqs, L.num_kv_heads, num_slots), -1, dtype=torch.int32, device=dev)
        self.slot_stamp = torch.full((L.num_seqs, L.num_kv_heads, num_slots), -1, dtype=torch.int64, device=dev)
        pool_dt = {kvs.KVS_F32: torch.float32, kvs.KVS_BF16: torch.bfloat16, kvs.KVS_FP8_E4M3: torch.uint8}[L.kv_dtype]
        self.hot_k = torch.zeros((units * num_slots, L.block_size, L.head_dim), dtype=pool_dt, device=dev)
        T = min(L.block_size, 32)  # V tiles: runs of T tokens, each channel-major
        self.hot_v = torch.zeros((units * num_slots, L.block_size // T, L.head_dim, T), dtype=pool_dt, device=dev)
        if L.quant_group:
            sshape = (units * num_slots, L.block_size, L.head_dim // L.quant_group)
            self.hot_ks = torch.ones(sshape, dtype=torch.float32, device=dev)
            self.hot_vs = torch.ones(sshape, dtype=torch.float32, device=dev)
        else:
            self.hot_ks = self.hot_vs = None
        self.miss_list = torch.empty((L.num_seqs, L.num_kv_heads, k), dtype=torch.int32, device=dev)
        self.miss_count = torch.empty((L.num_seqs, L.num_kv_heads), dtype=torch.int32, device=dev)
        self.out = torch.empty((L.num_seqs, L.num_q_heads, L.head_dim), dtype=torch.float32, device=dev)
        self.attn_ws = torch.zeros(max(kvs.kvs_attn_workspace_size(self.hot_layout, k), 1), dtype=torch.uint8, device=dev)
        self.sm_scale = 1.0 / math.sqrt(L.head_dim)

    def swap_in(self, step, sel, host_k, host_v, host_ks=None, host_vs=None, stream=None,
                live: kvs.HotLive | None = None):
        kvs.kvs_hot_lookup_swapin(self.host_layout, sel, self.k, self.ns, step, self.page_table,
                                  self.slot_owner, self.slot_stamp, host_k, host_v, host_ks, host_vs,
                                  self.hot_k, self.hot_v, self.hot_ks, self.hot_vs, self.miss_list,
                                  self.miss_count, stream, live=live)

    def lookup(self, step, sel, stream=None):
        """The page-table step alone (hits, miss list, LRU victims)."""
        kvs.kvs_hot_lookup(self.host_layout, sel, self.k, self.ns, step, self.page_table, self.slot_owner,
                           self.slot_stamp, self.miss_list, self.miss_count, stream)

    def copy(self, host_k, host_v, host_ks=None, host_vs=None, stream=None, live: kvs.HotLive | None = None):
        """The copy of the misses the last lookup listed (and, with `live`,
        of each sequence's newest block from the paged cache)."""
        kvs.kvs_hot_swapin(self.host_layout, self.k, self.ns, self.page_table, self.miss_list, self.miss_count,
                           host_k, host_v, host_ks, host_vs, self.hot_k, self.hot_v, self.hot_ks, self.hot_vs,
                           stream, live=live)

    def attend(self, q, sel, seq_lens, stream=None) -> torch.Tensor:
        kvs.kvs_sparse_decode_attn(self.hot_layout, kvs.KVS_TABLE_HOT, q, self.hot_k, self.hot_v,
                                   self.hot_ks, self.hot_vs, self.page_table, seq_lens, sel, self.k,
                                   self.sm_scale, self.out, self.attn_ws, stream)
        return self.out

    def run(self, step, sel, q, seq_lens, host_k, host_v, host_ks=None, host_vs=None, stream=None,
            live: kvs.HotLive | None = None):
        self.swap_in(step, sel, host_k, host_v, host_ks, host_vs, stream, live=live)
        return self.attend(q, sel, seq_lens, stream)


class HotPrefetchPipeline:
    """Hot-buffer decode steps over several layers whose selections are known
    ahead (the premise of selecting KV early, "SparDA…" §3–4): layer i+1's
    misses come in over the host link while layer i attends, so the copies
    leave the decode critical path ("KV 稀疏化" §7 names misses on that path
    as the cost of the hot buffer; "分块稀疏注意力与KV Cache量化…" §5.3 widens
    decode prefetch).

    Each layer has its own HotBufferStep.  lookup(i) runs layer i's
    page-table step (kvs_hot_lookup) on the compute stream; swapin(i) runs
    its copy (kvs_hot_swapin) on a copy stream, after that lookup;
    attend(i) waits for that copy.  step(i) keeps the lookups two layers
    ahead and the copies one layer ahead: the lookup (a chain of dependent
    reads, slow beside the HBM-saturating attention) then runs while an
    earlier copy is on the host link and is off the path between two
    copies, and the copy stream carries only copies, back to back.  Every
    lookup follows, on the compute stream, the earlier attentions of its
    buffer; with lookups two layers ahead that needs at least three
    buffers.  Both streams keep the default priority.  The copies run ahead
    of their layers' steps, so they take every block from the host tier: a
    decode loop that appends tokens (whose newest blocks the host tier does
    not hold yet) uses HotBufferStep with a live source instead."""

    def __init__(self, steps: list, device="cuda", copy_ahead: int = 2):
        if len(steps) < 3:
            raise ValueError("the pipeline needs at least three hot buffers")
        if copy_ahead not in (1, 2):
            raise ValueError("copy_ahead must be 1 or 2")
        self.hs = steps
        self.copy_ahead = copy_ahead
        dev = torch.device(device)
        self.copy_stream = torch.cuda.Stream(device=dev)
        self.looked = [torch.cuda.Event() for _ in steps]
        self.ready = [torch.cuda.Event() for _ in steps]
        self.next_lookup = self.next_copy = 0

    def lookup(self, i, step, sel):
        """Buffer i's page-table step on the current stream."""
        self.hs[i].lookup(step, sel)
        self.looked[i].record(torch.cuda.current_stream())

    def swapin(self, i, host_k, host_v, host_ks=None, host_vs=None):
        """Buffer i's copy on the copy stream, after its lookup."""
        s = self.copy_stream
        s.wait_event(self.looked[i])
        with torch.cuda.stream(s):
            self.hs[i].copy(host_k, host_v, host_ks, host_vs)
        self.ready[i].record(s)

    def prefetch(self, i, step, sel, host_k, host_v, host_ks=None, host_vs=None):
        """Buffer i's lookup and copy, issued now."""
        self.lookup(i, step, sel)
        self.swapin(i, host_k, host_v, host_ks, host_vs)

    def attend(self, i, q, sel, seq_lens) -> torch.Tensor:
        """Buffer i's attention on the current stream, after its copy."""
        torch.cuda.current_stream().wait_event(self.ready[i])
        return self.hs[i].attend(q, sel, seq_lens)

    def step(self, n, layer_of, lookup_args, host, q, sel, seq_lens) -> torch.Tensor:
        """Decode layer-step n of a sequence of steps numbered 0, 1, ...:
        step m runs buffer layer_of(m) with lookup_args(m) = (step, sel)
        for its lookup.  Issues the lookups up to step n+2 and the copies
        up to step n+1 that are not issued yet, then step n's attention."""
        while self.next_lookup <= n + 2:
            m = self.next_lookup
            self.lookup(layer_of(m), *lookup_args(m))
            self.next_lookup += 1
            # the copy's wait goes in right after the lookup's record: on this
            # stack a wait on an event can also wait for work the recording
            # stream received after the record
            while self.next_copy <= min(m, n + self.copy_ahead):
                self.swapin(layer_of(self.next_copy), *host)
                self.next_copy += 1
        return self.attend(layer_of(n), q, sel, seq_lens)


class CrossLayerDecode:
    """A decode step over a model's layers that selects once
    ("SparDA：把KV選擇提前一層…" §3.1, §4.1: a few shallow layers score the
    history, their scores are fused into one mask, and every deeper layer
    gathers the K/V that mask names, skipping its own selection).

    Predictor layer l < P appends its decode token, adds its exact block
    scores to the fused score (kvs_score_blocks with accumulate for l > 0,
    so the fused score is the sum over layers 0..l, added in layer order)
    and attends over the top-k of that sum (kvs_select_attn).  Every deeper
    layer appends its token (its K/V written, its summary kept current) and
    attends over the last predictor layer's selection, in one call
    (kvs_append_sparse_decode_attn: one launch for bf16 K/V): it reads no
    summaries and scores nothing.  Block ids are logical positions, so each layer gathers its own
    pages through its own block table.  All layers share seq_lens."""

    def __init__(self, layout: kvs.Layout, k: int, num_layers: int, predictor_layers: int, device="cuda"):
        if not 1 <= predictor_layers <= num_layers:
            raise ValueError("need 1 <= predictor_layers <= num_layers")
        L = self.layout = layout
        self.k, self.n, self.P = k, num_layers, predictor_layers
        dev = torch.device(device)
        self.fused = torch.empty((L.num_seqs, L.num_kv_heads, L.max_blocks), dtype=torch.float64, device=dev)
        self.sel = torch.empty((L.num_seqs, L.num_kv_heads, k), dtype=torch.int32, device=dev)
        self.out = torch.empty((num_layers, L.num_seqs, L.num_q_heads, L.head_dim), dtype=torch.float32, device=dev)
        self.attn_ws = torch.zeros(max(kvs.kvs_attn_workspace_size(L, k), 1), dtype=torch.uint8, device=dev)
        self.sm_scale = 1.0 / math.sqrt(L.head_dim)
        self._first = kvs.SelectOpts()
        self._more = kvs.SelectOpts(accumulate=True)

    def layer(self, l: int, q, tok: kvs.AppendArgs, seq_lens, summaries, stream=None) -> torch.Tensor:
        """Layer l of the step (layers run in order 0, 1, ...); returns its
        attention output [B][Hq][D]."""
        L, k = self.layout, self.k
        if l < self.P:
            kvs.kvs_score_blocks(L, q, summaries, seq_lens, self._more if l > 0 else self._first, tok, self.fused,
                                 None, stream)
            kvs.kvs_select_attn(L, q, tok.k_pool, tok.v_pool, tok.k_scales, tok.v_scales, tok.block_table,
                                seq_lens, self.fused, k, 1, self.sel, self.sm_scale, self.out[l], self.attn_ws,
                                stream)
        else:
            kvs.kvs_append_sparse_decode_attn(L, tok, summaries, q, seq_lens, self.sel, k, self.sm_scale,
                                              self.out[l], self.attn_ws, stream)
        return self.out[l]

    def run(self, qs, toks, seq_lens, summaries, stream=None) -> torch.Tensor:
        """The whole step: per-layer queries, token appends and summaries
        (lists of num_layers); returns out [num_layers][B][Hq][D]."""
        for l in range(self.n):
            self.layer(l, qs[l], toks[l], seq_lens, summaries[l], stream)
        return self.out
