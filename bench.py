"""Decode-step benchmark of query-aware block-sparse attention on one MI355X.

A step is one decode layer-step of the whole path over one batch: append
every sequence's decode token to the paged cache and fold it into its
block's summary while scoring every block (kvs_score_blocks), then attend
over the top-k blocks, each attention workgroup selecting its unit's blocks
from the scores itself (kvs_select_attn: split partials + merge).  The
appended token is the one the cache already holds at that position, so the
replayed step leaves the cache as it was.  The
default workload is 8 sequences x 32 query / 4 KV heads, head dim 128, 32768
tokens of bf16 K/V in 64-token pages, k = 128 of 512 blocks, over 32 layer
instances with their own buffers (step i uses instance i mod 32, so no step
re-reads data an earlier step left in the 256 MB last-level cache).  The
layer sweep (every instance in order, as a decoder runs its layers) is
captured once into a HIP graph and the timed loop replays it.

Prints one JSON line.  Metric: decode query-tokens/s/layer = B / t(step),
with the achieved HBM GB/s of the step and a roofline entry for the dominant
kernel (the sparse attention) timed with HIP events on its own stream, plus
the CPU oracle's rate on a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--parts P] [--no-cpu] [--cpu-steps N]

--parts P cuts the batch into P slices of sequences whose kernel chains run
concurrently on their own streams inside the step (the units never interact).
The per-phase times in "phase_us" are whole-batch, one-chain runs of each
phase alone.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode query-tokens/s/layer + achieved HBM GB/s (% peak), top-25% @32K ctx"
PEAK_HBM_GBPS = 8000.0


def algorithmic_bytes(w, summ_elem: int, kv_elem: int, q_elem: int) -> dict:
    """Bytes one layer-step must move: the summaries of every block, the
    selected K/V tiles (and fp8 scales), q, the fp32 output, and the decode
    token's append (its K and V read and written, with fp8 scales, and its
    block's summary row read and written)."""
    units = w.B * w.Hkv
    summ = units * w.nb * 2 * w.D * summ_elem
    tile = w.S * w.D * kv_elem
    kv = units * w.k * 2 * tile
    scales = units * w.k * 2 * w.S * (w.D // w.quant_group) * 4 if w.quant_group else 0
    q = w.B * w.Hq * w.D * q_elem
    out = w.B * w.Hq * w.D * 4
    tok = 2 * w.D * kv_elem + (2 * (w.D // w.quant_group) * 4 if w.quant_group else 0)  # K and V of one token
    append = units * (2 * tok + 2 * 2 * w.D * summ_elem)
    return {"summaries": summ, "kv": kv, "scales": scales, "q": q, "out": out, "append": append,
            "attention": kv + scales + q + out,
            "scores": units * w.nb * 8,
            "step": summ + kv + scales + q + out + append}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--parts", type=int, default=1,
                    help="batch slices run as concurrent chains within a step (1 = one chain)")
    ap.add_argument("--layers", type=int, default=0,
                    help="layer instances to rotate through (default: the workload's own count)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference kernel "
                         "for scaling HBM byte counters) and exit")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--prefetch", action="store_true",
                    help="hot-buffer workload: swap in the next layer's misses on a second stream while the "
                         "current layer attends (selections known one layer ahead)")
    ap.add_argument("--copy-ahead", type=int, default=2, choices=(1, 2),
                    help="hot-buffer prefetch: copies issued 1 or 2 layers ahead (page-table steps 2 ahead)")
    ap.add_argument("--selection-study", action="store_true",
                    help="instead of the step benchmark: selection churn and hot-buffer misses over a "
                         "drifting query, plain / smoothed / recent window / both (one JSON line)")
    ap.add_argument("--separate-topk", action="store_true",
                    help="time the step with the top-k as a launch of its own (kvs_select_topk_ex + "
                         "kvs_sparse_decode_attn) instead of inside the attention launch")
    ap.add_argument("--cpu-steps", type=int, default=6, help="layer-steps in the CPU oracle sample (about 2 s each)")
    ap.add_argument("--reuse", type=int, default=0, metavar="P",
                    help="also time a decode step over all layer instances that selects once: layers 0..P-1 "
                         "score (fused) and select, every other layer attends over that selection")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path: (sequence, KV head) units are independent, so several GPUs would "
              "each run this same step on their share of the sequences.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from query_aware_sparse_kvs_amd import kvs, synth
    from query_aware_sparse_kvs_amd.step import SparseDecodeStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return 0
    w = synth.WORKLOADS[args.workload]
    if args.selection_study:
        return selection_study(args, w, dev)
    if w.hot_slots:
        return bench_hot(args, w, dev)
    code = kvs.DTYPE_CODE
    L = kvs.Layout(w.B, w.Hq, w.Hkv, w.D, w.S, w.nb, w.B * w.nb, code[w.q_dtype], code[w.kv_dtype],
                   w.quant_group)
    n_layers = args.layers if args.layers > 0 else w.layers
    print(f"[bench] workload {w.name}: building {n_layers} layer instance(s)", file=sys.stderr, flush=True)

    layers = []
    steps = []
    for li in range(n_layers):
        inp = synth.make_inputs(w, dev, layer=li)
        st = SparseDecodeStep(L, w.k, dev, parts=args.parts)
        summ = st.new_summaries(dev)
        st.prefill_summaries(inp["k_pool"], inp["k_scales"], inp["block_table"], inp["seq_lens"], summ)
        newest = ((inp["seq_lens"] + w.S - 1) // w.S - 1).to(torch.int32)
        nt = synth.newest_tokens(w, inp)
        tok = kvs.AppendArgs(k_new=nt["k_new"], v_new=nt["v_new"], k_new_scales=nt["k_new_scales"],
                             v_new_scales=nt["v_new_scales"], block_table=inp["block_table"],
                             k_pool=inp["k_pool"], v_pool=inp["v_pool"], k_scales=inp["k_scales"],
                             v_scales=inp["v_scales"])
        mean = torch.empty((w.B, w.Hkv, w.nb, w.D), dtype=torch.float32, device=dev)
        kvs.kvs_build_summaries_ex(L, kvs.KVS_SUMM_MEAN, inp["k_pool"], inp["k_scales"], inp["block_table"],
                                   inp["seq_lens"], None, L.max_blocks, mean)
        layers.append(dict(inp=inp, summ=summ, newest=newest, tok=tok, nt=nt, mean=mean))
        steps.append(st)
    torch.cuda.synchronize()
    assert kvs.kvs_device_errors() == 0

    def run_select_append(i):
        d, st = layers[i], steps[i]
        inp = d["inp"]
        kvs.kvs_select_topk_append(L, inp["q"], inp["k_pool"], inp["k_scales"], inp["block_table"],
                                   inp["seq_lens"], d["summ"], w.k, st.sel, None, st.select_ws)

    # where the library selects on the matrix cores, the separate selection
    # launch is the cheaper step (the in-attention top-k needs every exact score)
    matrix_cores = kvs.kvs_select_uses_matrix_cores(L, w.k)

    def run_append_select(i):
        d, st = layers[i], steps[i]
        inp = d["inp"]
        kvs.kvs_select_topk_ex(L, inp["q"], d["summ"], inp["seq_lens"], w.k, None, d["tok"], st.sel, None,
                               st.select_ws)

    def run_select(i):
        d, st = layers[i], steps[i]
        inp = d["inp"]
        kvs.kvs_select_topk(L, inp["q"], d["summ"], inp["seq_lens"], w.k, st.sel, None, st.select_ws)

    def run_attn(i):
        d, st = layers[i], steps[i]
        inp = d["inp"]
        kvs.kvs_sparse_decode_attn(L, kvs.KVS_TABLE_PAGED, inp["q"], inp["k_pool"], inp["v_pool"],
                                   inp["k_scales"], inp["v_scales"], inp["block_table"], inp["seq_lens"],
                                   st.sel, w.k, st.sm_scale, st.out, st.attn_ws)

    def run_step(i):
        d, st = layers[i], steps[i]
        inp = d["inp"]
        if args.parts > 1:  # the summary-rebuild chain, cut into concurrent batch slices
            st.run(inp["q"], inp["k_pool"], inp["v_pool"], inp["k_scales"], inp["v_scales"], inp["block_table"],
                   inp["seq_lens"], d["summ"])
        elif args.separate_topk or matrix_cores:
            st.run_decode(inp["q"], d["tok"], inp["seq_lens"], d["summ"])
        else:
            st.run_decode_fused(inp["q"], d["tok"], inp["seq_lens"], d["summ"])

    def run_score(i):
        d, st = layers[i], steps[i]
        inp = d["inp"]
        kvs.kvs_score_blocks(L, inp["q"], d["summ"], inp["seq_lens"], None, d["tok"], st.scores, None)

    mean_opts = kvs.SelectOpts(summary_kind=kvs.KVS_SUMM_MEAN)

    def run_score_mean(i):
        d, st = layers[i], steps[i]
        inp = d["inp"]
        kvs.kvs_score_blocks(L, inp["q"], d["mean"], inp["seq_lens"], mean_opts, None, st.scores, None)
        kvs.kvs_select_attn(L, inp["q"], inp["k_pool"], inp["v_pool"], inp["k_scales"], inp["v_scales"],
                            inp["block_table"], inp["seq_lens"], st.scores, w.k, 1, st.sel, st.sm_scale, st.out,
                            st.attn_ws)

    def run_select_attn(i):
        d, st = layers[i], steps[i]
        inp = d["inp"]
        kvs.kvs_select_attn(L, inp["q"], inp["k_pool"], inp["v_pool"], inp["k_scales"], inp["v_scales"],
                            inp["block_table"], inp["seq_lens"], st.scores, w.k, 1, st.sel, st.sm_scale, st.out,
                            st.attn_ws)

    def graph_of(fn, layer_ids):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in layer_ids:
                fn(i)
        return g

    def capture(fn):
        """One graph over every layer instance in order (as a decoder runs its
        layers) and, when the warm-up or timed step count is not a multiple of
        the layer count, one graph over the first (count mod layers)
        instances: any step count then replays whole graphs of the same layer
        sequence, with no per-step graph launches."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(n_layers):
                fn(i)  # eager warm-up (also initialises the library's per-device state)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        sweep = graph_of(fn, range(n_layers))
        part = {}
        for count in (args.steps, args.warmup):
            r = count % n_layers
            if r and r not in part:
                part[r] = graph_of(fn, range(r))
        return sweep, part

    def replay(graphs, K):
        sweep, part = graphs
        for _ in range(K // n_layers):
            sweep.replay()
        if K % n_layers:
            part[K % n_layers].replay()

    def timed(graphs, K, W):
        replay(graphs, W)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        replay(graphs, K)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / 1e3, wall

    step_graphs = capture(run_step)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} layer-steps after {args.warmup} warm-up", file=sys.stderr, flush=True)
    t_step, wall_step = timed(step_graphs, args.steps, args.warmup)
    phase = {"step_sweep_us": t_step / args.steps * 1e6}
    # distribution: every layer-step graph replayed alone between two HIP
    # events (the sweep above is the throughput figure; these include the
    # launch of one graph and one event pair per step)
    single = [graph_of(run_step, [i]) for i in range(n_layers)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        single[i % n_layers].replay()
        e1.record()
    torch.cuda.synchronize()
    del single
    per = np.sort(np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]))
    pct = {f"p{q}": round(float(np.percentile(per, q)), 3) for q in (10, 50, 90)}
    # per-phase graphs: the dominant kernel (attention) for the roofline entry,
    # the token append with the selection as the step runs it, the selection
    # alone (the append's cost is the difference), and the selection with a
    # rebuild of the newest block's summary from its K tile instead
    for name, fn in (("score_blocks", run_score), ("select_attn", run_select_attn),
                     ("mean_summaries_step", run_score_mean),
                     ("append_select", run_append_select), ("select_topk_only", run_select),
                     ("select_topk_rebuild", run_select_append), ("attention", run_attn)):
        t, _ = timed(capture(fn), args.steps, args.warmup)
        phase[name] = t / args.steps * 1e6
    reuse = None
    if args.reuse > 0:
        reuse = time_reuse(args, w, L, layers, steps, n_layers, capture, timed, phase)
    # the roofline entry is for the step's dominant call: the attention with
    # its own selection (or, with --separate-topk, the attention alone)
    fused = not args.separate_topk and not matrix_cores and args.parts == 1
    t_attn = phase["select_attn" if fused else "attention"] * 1e-6 * args.steps
    torch.cuda.synchronize()
    assert kvs.kvs_device_errors() == 0, "kernels raised device error flags"

    summ_elem = 2 if w.kv_dtype == "bf16" else 4
    kv_elem = {"f32": 4, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    q_elem = 4 if w.q_dtype == "f32" else 2
    by = algorithmic_bytes(w, summ_elem, kv_elem, q_elem)
    sec_per_step = t_step / args.steps
    attn_sec = t_attn / args.steps
    value = w.B / sec_per_step
    step_gbps = by["step"] / sec_per_step / 1e9
    attn_bytes = by["attention"] + (by["scores"] if fused else 0)
    attn_gbps = attn_bytes / attn_sec / 1e9
    attn_kernel = {"bf16": "attn_mfma_kernel", "e4m3": "attn_mfma8_kernel"}.get(w.kv_dtype, "attn_valu_kernel")

    cpu = parity = None
    if not args.no_cpu:
        # each sampled layer's GPU results from one more step (the phase
        # graphs above leave other phases' results in the step buffers)
        gpu_results = []
        for li in range(min(args.cpu_steps, n_layers)):
            run_step(li)
            torch.cuda.synchronize()
            gpu_results.append((steps[li].sel.cpu().numpy(), steps[li].out.cpu().numpy()))
        assert kvs.kvs_device_errors() == 0, "kernels raised device error flags"
        cpu, parity = cpu_baseline(w, layers, args.cpu_steps, gpu_results)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_per_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "context": w.L, "block": w.S, "top_k_blocks": w.k,
                   "kv_storage": w.kv_dtype, "q_storage": w.q_dtype, "layer_instances": n_layers,
                   "graph_replay": True, "concurrent_batch_slices": len(steps[0].slices),
                   "topk": "inside the attention launch" if fused else "separate launch"},
        "phase_us": {k: round(v, 3) for k, v in phase.items() if k != "step_sweep_us"},
        "step_us_percentiles": pct,
        "step_bytes": by["step"],
        "step_GBps": round(step_gbps, 1),
        "step_hbm_frac": round(step_gbps / PEAK_HBM_GBPS, 4),
        "roofline": {"bound": "hbm",
                     "kernel": ((f"kvs_select_attn (self-selecting {attn_kernel} + merge_kernel)" if fused else
                                 f"kvs_sparse_decode_attn ({attn_kernel} + merge_kernel)")
                                if kvs.kvs_attn_num_splits(L, w.k) > 1 else
                                (f"kvs_select_attn (self-selecting {attn_kernel})" if fused else
                                 f"kvs_sparse_decode_attn ({attn_kernel})")),
                     "achieved": round(attn_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(w.name, "select_attn" if fused else "attention"),
                     "bytes_per_launch": attn_bytes, "us_per_launch": round(attn_sec * 1e6, 3)},
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "cross_layer_reuse": reuse,
        "wall_s_timed_region": round(wall_step, 4),
    }
    print(json.dumps(result), flush=True)
    return 0


def time_reuse(args, w, L, layers, steps, n_layers, capture, timed, phase) -> dict:
    """Cross-layer selection reuse ("SparDA…" §3.1, §4.1): one decode step
    over all layer instances, in order, where layers 0..P-1 add their block
    scores into one fused score and attend over its top-k, and every other
    layer appends its token and attends over that selection without reading
    its summaries.  Timed as whole model steps (graph sweeps), reported per
    layer beside the step without reuse."""
    from query_aware_sparse_kvs_amd.step import CrossLayerDecode
    P = min(args.reuse, n_layers)
    cl = CrossLayerDecode(L, w.k, n_layers, P, steps[0].sel.device)

    def run_layer(i):
        d = layers[i]
        inp = d["inp"]
        cl.layer(i, inp["q"], d["tok"], inp["seq_lens"], d["summ"])

    model_steps = max(1, args.steps // n_layers)
    K, W = model_steps * n_layers, max(1, args.warmup // n_layers) * n_layers
    t, _ = timed(capture(run_layer), K, W)
    per_layer = t / K
    summ_elem = 2 if w.kv_dtype == "bf16" else 4
    kv_elem = {"f32": 4, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    by = algorithmic_bytes(w, summ_elem, kv_elem, 4 if w.q_dtype == "f32" else 2)
    # deeper layers read no summaries
    model_bytes = n_layers * by["step"] - (n_layers - P) * by["summaries"]
    full = phase.get("step_sweep_us")
    return {"predictor_layers": P, "layers": n_layers, "model_steps_timed": model_steps,
            "us_per_layer": round(per_layer * 1e6, 3),
            "query_tokens_per_s_per_layer": round(w.B / per_layer, 1),
            "GBps": round(model_bytes / n_layers / per_layer / 1e9, 1),
            "us_per_layer_without_reuse": None if full is None else round(full, 3)}


def bench_hot(args, w, dev) -> int:
    """Hot-buffer layer-step (page "KV 稀疏化", §7): page-table lookup, LRU
    slot assignment and swap-in of the missed blocks from pinned host memory,
    then attention through the hot table.  Each layer instance has its own
    hot buffer (so the 256 MB last-level cache cannot hold them all) and
    steps through the same seeded drift stream: after a warm start from the
    computed top-k, every step misses `drift` blocks per (sequence, KV head).
    Launched eagerly (the step is bound by the host link, not by launches)."""
    import torch

    from query_aware_sparse_kvs_amd import kvs, synth
    from query_aware_sparse_kvs_amd.step import HotBufferStep, SparseDecodeStep

    code = kvs.DTYPE_CODE
    L = kvs.Layout(w.B, w.Hq, w.Hkv, w.D, w.S, w.nb, w.B * w.nb, code[w.q_dtype], code[w.kv_dtype],
                   w.quant_group)
    n_layers = args.layers if args.layers > 0 else 8
    print(f"[bench] workload {w.name}: {n_layers} hot buffers of {w.hot_slots} slots per unit",
          file=sys.stderr, flush=True)
    inp = synth.make_inputs(w, dev, layer=0)
    st = SparseDecodeStep(L, w.k, dev)
    summ = st.new_summaries(dev)
    st.prefill_summaries(inp["k_pool"], inp["k_scales"], inp["block_table"], inp["seq_lens"], summ)
    kvs.kvs_select_topk(L, inp["q"], summ, inp["seq_lens"], w.k, st.sel, None, st.select_ws)
    sel0 = st.sel.cpu().numpy()
    per_phase = (args.warmup + args.steps) // n_layers + 2
    stream = synth.drift_selections(sel0, w.nb, 4 * per_phase, w.drift, seed=w.seed)
    sels = torch.from_numpy(stream).to(dev)
    # host tier [B][Hkv][MB][S][D] (V tiles [D][S]), pinned and shared by the layer instances
    pages = inp["block_table"].long().cpu()
    host = [None if inp[n] is None else inp[n].cpu()[pages].transpose(1, 2).contiguous().pin_memory()
            for n in ("k_pool", "v_pool", "k_scales", "v_scales")]
    hs = [HotBufferStep(L, w.k, w.hot_slots, dev) for _ in range(n_layers)]
    for h in hs:  # warm start: the first selection fills every slot
        h.run(0, sels[0], inp["q"], inp["seq_lens"], *host)
    torch.cuda.synchronize()
    assert kvs.kvs_device_errors() == 0
    m = [1] * n_layers  # next stream index per layer instance

    def swap(i):
        h = hs[i % n_layers]
        t = m[i % n_layers]
        h.swap_in(t, sels[t], *host)
        return h, t

    def step(i):
        h, t = swap(i)
        h.attend(inp["q"], sels[t], inp["seq_lens"])
        m[i % n_layers] += 1

    def only_swap(i):
        swap(i)
        m[i % n_layers] += 1

    def only_attend(i):
        h = hs[i % n_layers]
        h.attend(inp["q"], sels[m[i % n_layers] - 1], inp["seq_lens"])

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            fn(args.warmup + i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / args.steps

    t_step = timed(step)
    t_swap = timed(only_swap)
    t_attn = timed(only_attend)
    t_pipe = None
    if args.prefetch:
        from query_aware_sparse_kvs_amd.step import HotPrefetchPipeline
        pipe = HotPrefetchPipeline(hs, dev, copy_ahead=args.copy_ahead)
        base = list(m)  # each buffer's next stream entry
        layer_of = lambda i: i % n_layers
        index_of = lambda i: base[i % n_layers] + i // n_layers
        lookup_args = lambda i: (index_of(i), sels[index_of(i)])

        def piped(i):  # layer i attends while layer i+1's misses come in
            pipe.step(i, layer_of, lookup_args, host, inp["q"], sels[index_of(i)], inp["seq_lens"])

        t_pipe = timed(piped)
        torch.cuda.synchronize()
    miss = hs[0].miss_count.sum().item()
    assert kvs.kvs_device_errors() == 0, "kernels raised device error flags"
    # pinned host -> device copy rate of the runtime, for reference
    src = torch.empty(256 << 20, dtype=torch.uint8).pin_memory()
    dst = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d = 4 * (256 << 20) / (e0.elapsed_time(e1) / 1e3) / 1e9

    kv_elem = {"f32": 4, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    tile = w.S * w.D * kv_elem + (w.S * (w.D // w.quant_group) * 4 if w.quant_group else 0)
    link_bytes = int(miss) * 2 * tile                       # K and V of every missed block
    units = w.B * w.Hkv
    attn_bytes = units * w.k * 2 * tile + w.B * w.Hq * w.D * (2 + 4)
    link_gbps = link_bytes / t_swap / 1e9
    t_best = t_pipe if t_pipe is not None else t_step
    result = {
        "metric": METRIC,
        "value": round(w.B / t_best, 1),
        "unit": "query-tokens/s/layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_best * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
                   "context": w.L, "block": w.S, "top_k_blocks": w.k, "hot_slots": w.hot_slots,
                   "drift_per_step": w.drift, "kv_storage": w.kv_dtype, "layer_instances": n_layers,
                   "graph_replay": False, "prefetch_next_layer": bool(args.prefetch)},
        "phase_us": {"swap_in": round(t_swap * 1e6, 3), "attention": round(t_attn * 1e6, 3),
                     "sequential_step": round(t_step * 1e6, 3),
                     "prefetched_step": None if t_pipe is None else round(t_pipe * 1e6, 3)},
        "misses_per_step": int(miss),
        "roofline": {"bound": "host-link", "kernel": "kvs_hot_lookup_swapin",
                     "achieved": round(link_gbps, 2), "peak": 64.0, "unit": "GB/s",
                     "frac": round(link_gbps / 64.0, 4), "traffic": None,
                     "bytes_per_launch": link_bytes, "us_per_launch": round(t_swap * 1e6, 3),
                     "peak_note": "PCIe Gen5 x16, one direction",
                     "pinned_h2d_copy_GBps": round(h2d, 2)},
        "attention_hbm_GBps": round(attn_bytes / t_attn / 1e9, 1),
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


def selection_study(args, w, dev) -> int:
    """How stable the selection is from one decode step to the next ("SparDA…"
    §6.1 smooths the scores so that the mask stops jumping; §4.2 keeps a
    recent window), and what that does to a hot buffer of k slots per unit
    ("KV 稀疏化" §7): every block that enters the selection is a miss copied
    in over the host link.  The query drifts as a seeded random walk
    q <- rho*q + sqrt(1-rho^2)*noise (rho = 0.95), the stand-in for a
    decode's successive queries; the cache is the workload's first layer.
    For each variant the steps run eagerly: kvs_select_topk_ex (exact
    scores, smoothing state kept across steps), kvs_hot_lookup_swapin,
    attention through the hot table."""
    import torch

    from query_aware_sparse_kvs_amd import kvs, synth
    from query_aware_sparse_kvs_amd.step import HotBufferStep, SparseDecodeStep

    code = kvs.DTYPE_CODE
    L = kvs.Layout(w.B, w.Hq, w.Hkv, w.D, w.S, w.nb, w.B * w.nb, code[w.q_dtype], code[w.kv_dtype],
                   w.quant_group)
    inp = synth.make_inputs(w, dev, layer=0)
    st = SparseDecodeStep(L, w.k, dev)
    summ = st.new_summaries(dev)
    st.prefill_summaries(inp["k_pool"], inp["k_scales"], inp["block_table"], inp["seq_lens"], summ)
    pages = inp["block_table"].long().cpu()
    host = [None if inp[n] is None else inp[n].cpu()[pages].transpose(1, 2).contiguous().pin_memory()
            for n in ("k_pool", "v_pool", "k_scales", "v_scales")]
    steps, rho = 64, 0.95
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed * 7919 + 11)
    qs = [inp["q"].float()]
    for _ in range(steps):
        noise = torch.randn(qs[-1].shape, generator=g, device=dev)
        qs.append(rho * qs[-1] + math.sqrt(1.0 - rho * rho) * noise)
    qs = [x.to(inp["q"].dtype).contiguous() for x in qs]
    variants = {"plain": (1, False), "ema0.7": (1, True), "window8": (8, False), "window8+ema0.7": (8, True),
                "mean-summaries": (1, False)}
    mean = torch.empty((w.B, w.Hkv, w.nb, w.D), dtype=torch.float32, device=dev)
    kvs.kvs_build_summaries_ex(L, kvs.KVS_SUMM_MEAN, inp["k_pool"], inp["k_scales"], inp["block_table"],
                               inp["seq_lens"], None, L.max_blocks, mean)
    units = w.B * w.Hkv
    kv_elem = {"f32": 4, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    tile = w.S * w.D * kv_elem + (w.S * (w.D // w.quant_group) * 4 if w.quant_group else 0)
    res = {}
    for name, (recent, ema) in variants.items():
        state = torch.full((w.B, w.Hkv, w.nb), float("nan"), dtype=torch.float64, device=dev)
        kind = kvs.KVS_SUMM_MEAN if name == "mean-summaries" else kvs.KVS_SUMM_MINMAX
        opts = kvs.SelectOpts(recent_blocks=recent, use_ema=ema, ema_alpha=0.7, ema_state=state if ema else None,
                              summary_kind=kind)
        table = mean if kind == kvs.KVS_SUMM_MEAN else summ
        hs = HotBufferStep(L, w.k, w.k, dev)
        misses = []
        t_sel = t_swap = t_attn = 0.0
        for t, q in enumerate(qs):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record()
            kvs.kvs_select_topk_ex(L, q, table, inp["seq_lens"], w.k, opts, None, st.sel, None, st.select_ws)
            ev[1].record()
            hs.swap_in(t, st.sel, *host)
            ev[2].record()
            hs.attend(q, st.sel, inp["seq_lens"])
            ev[3].record()
            torch.cuda.synchronize()
            if t > 0:  # step 0 fills the empty buffer
                misses.append(int(hs.miss_count.sum().item()))
                t_sel += ev[0].elapsed_time(ev[1]) / 1e3
                t_swap += ev[1].elapsed_time(ev[2]) / 1e3
                t_attn += ev[2].elapsed_time(ev[3]) / 1e3
        n = len(misses)
        res[name] = {"misses_per_step": round(sum(misses) / n, 2),
                     "misses_per_unit_step": round(sum(misses) / n / units, 3),
                     "host_link_bytes_per_step": int(sum(misses) / n * 2 * tile),
                     "select_us": round(t_sel / n * 1e6, 2), "swap_in_us": round(t_swap / n * 1e6, 2),
                     "attention_us": round(t_attn / n * 1e6, 2)}
    assert kvs.kvs_device_errors() == 0, "kernels raised device error flags"
    print(json.dumps({"study": "selection stability over a drifting query", "workload": w.name,
                      "steps": steps, "rho": rho, "k": w.k, "hot_slots_per_unit": w.k, "units": units,
                      "launch": "eager, per call HIP events", "variants": res}), flush=True)
    return 0


ATTN_SOURCES = ("query_aware_sparse_kvs_amd/csrc/kvs_attn.hip", "query_aware_sparse_kvs_amd/csrc/kvs_internal.h",
                "query_aware_sparse_kvs_amd/csrc/kvs_topk.h")


def attn_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, call: str):
    """HBM bytes per call of `call` (attention: kvs_sparse_decode_attn;
    select_attn: kvs_select_attn; both kernels of the call) from the counter
    summary in profiles/, scaled by the copy-kernel calibration recorded
    there; None when there is none for this workload or the attention sources
    have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{call}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    if rec.get("attention_sources_sha256") != attn_source_digest():
        return None
    try:
        return int(rec["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def host_info() -> dict:
    """The host the CPU baseline runs on: logical CPUs, the ones this process
    may use, and the CPU model from /proc/cpuinfo."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0))}


NEAR_TIE = 1e-4  # the acceptance band: (k-2)-th and (k-1)-th free candidate scores


def near_tie_units(W, lens, S, k) -> int:
    """Units whose (k-2)-th and (k-1)-th best free candidates score within
    NEAR_TIE relative of each other (there a selection may differ)."""
    n = 0
    for b, L in enumerate(lens):
        nb = (int(L) + S - 1) // S
        if nb <= k or k < 3:
            continue
        for g in range(W.shape[1]):
            c = np.sort(W[b, g, 1:nb - 1])[::-1]
            a, z = c[k - 3], c[k - 2]
            if abs(a - z) <= NEAR_TIE * max(abs(a), abs(z)):
                n += 1
    return n


def cpu_baseline(w, layers, n_steps, gpu_results, max_threads=16):
    """The oracle (fp64, as written) on `n_steps` whole layer-steps of the
    same workload -- decode-token append (with its block's summary), bounds,
    selection, sparse attention -- run once on one thread and once fanned out
    over the independent (sequence, KV head) units on up to `max_threads`
    host cores (the oracle's ctypes calls release the interpreter lock).  The
    one-thread run's selections and outputs are also compared with the GPU's
    (`gpu_results`: per sampled layer, its sel and out after one step)."""
    import concurrent.futures as cf

    import torch

    import oracle
    code = {"f32": oracle.KV_F32, "bf16": oracle.KV_BF16, "e4m3": oracle.KV_E4M3}[w.kv_dtype]
    OL = oracle.Layout(w.B, w.Hq, w.Hkv, w.D, w.S, w.nb, w.B * w.nb, code, w.quant_group)
    n_steps = max(1, min(n_steps, len(layers)))
    sm = 1.0 / math.sqrt(w.D)

    def host_np(t):
        t = t.cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    host = []
    for li in range(n_steps):
        inp = layers[li]["inp"]
        h = {n: host_np(inp[n]) for n in ("k_pool", "v_pool")}
        for n in ("k_scales", "v_scales"):
            h[n] = None if inp[n] is None else inp[n].cpu().numpy()
        h["table"] = inp["block_table"].cpu().numpy()
        h["lens"] = inp["seq_lens"].cpu().numpy()
        h["q"] = inp["q"].double().cpu().numpy()
        nt = layers[li]["nt"]
        for n in ("k_new", "v_new"):
            h[n] = host_np(nt[n])
        for n in ("k_new_scales", "v_new_scales"):
            h[n] = None if nt[n] is None else nt[n].cpu().numpy()
        # prefill-time summaries of every block, built by the oracle (untimed)
        h["summ"] = oracle.summaries(OL, h["k_pool"], h["k_scales"], h["table"], h["lens"])
        # per-KV-head copies of the pools for the fan-out (untimed)
        for n in ("k_pool", "v_pool", "k_scales", "v_scales"):
            h[n + "_h"] = None if h[n] is None else [np.ascontiguousarray(h[n][:, g:g + 1]) for g in range(w.Hkv)]
        h["summ_u"] = {(b, g): np.ascontiguousarray(h["summ"][b:b + 1, g:g + 1])
                       for b in range(w.B) for g in range(w.Hkv)}
        host.append(h)

    def layer_step(h):
        """The oracle's layer-step for the whole batch."""
        oracle.append_token(OL, h["k_new"], h["v_new"], h["k_new_scales"], h["v_new_scales"], h["table"],
                            h["lens"], h["k_pool"], h["v_pool"], h["k_scales"], h["v_scales"], h["summ"])
        W = oracle.bounds(OL, h["q"], h["summ"], h["lens"])
        sel = oracle.select(OL, W, h["lens"], w.k)
        out = oracle.sparse_attn(OL, h["q"], h["k_pool"], h["v_pool"], h["k_scales"], h["v_scales"], h["table"],
                                 h["lens"], sel, sm)
        return W, sel, out

    def unit_step(h, b, g):
        """The same for one (sequence, KV head) unit, on its head's pools."""
        Lu = oracle.Layout(1, w.G, 1, w.D, w.S, w.nb, w.B * w.nb, code, w.quant_group)
        r, hs = slice(b, b + 1), slice(g * w.G, (g + 1) * w.G)
        pick = lambda n: None if h[n] is None else np.ascontiguousarray(h[n][r, g:g + 1])
        per = lambda n: None if h[n + "_h"] is None else h[n + "_h"][g]
        summ = h["summ_u"][(b, g)]
        oracle.append_token(Lu, pick("k_new"), pick("v_new"), pick("k_new_scales"), pick("v_new_scales"),
                            h["table"][r], h["lens"][r], per("k_pool"), per("v_pool"), per("k_scales"),
                            per("v_scales"), summ)
        q = np.ascontiguousarray(h["q"][r, hs])
        W = oracle.bounds(Lu, q, summ, h["lens"][r])
        sel = oracle.select(Lu, W, h["lens"][r], w.k)
        return sel, oracle.sparse_attn(Lu, q, per("k_pool"), per("v_pool"), per("k_scales"), per("v_scales"),
                                       h["table"][r], h["lens"][r], sel, sm)

    print(f"[bench] CPU oracle on {n_steps} layer-step(s), one thread", file=sys.stderr, flush=True)
    res = []
    t0 = time.perf_counter()
    for h in host:
        res.append(layer_step(h))
    dt1 = time.perf_counter() - t0
    units = w.B * w.Hkv
    threads = max(1, min(len(os.sched_getaffinity(0)), max_threads, units))
    print(f"[bench] CPU oracle on {n_steps} layer-step(s), {units} units per step over {threads} threads",
          file=sys.stderr, flush=True)
    tasks = [(li, b, g) for li in range(n_steps) for b in range(w.B) for g in range(w.Hkv)]
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        fan = list(ex.map(lambda t: unit_step(host[t[0]], t[1], t[2]), tasks))
    dtn = time.perf_counter() - t0
    # the fan-out computes the same thing unit by unit
    for (li, b, g), (sel_u, out_u) in zip(tasks, fan):
        assert np.array_equal(sel_u[0, 0], res[li][1][b, g]), "oracle fan-out selection differs"
        assert np.array_equal(out_u[0], res[li][2][b, g * w.G:(g + 1) * w.G]), "oracle fan-out output differs"

    # parity of the GPU's step against the one-thread oracle run
    ties = differ = differ_outside = 0
    err = num = den = 0.0
    for li, (W, o_sel, o_out) in enumerate(res):
        g_sel, g_out = gpu_results[li]
        lens = host[li]["lens"]
        ties += near_tie_units(W, lens, w.S, w.k)
        bad = ~np.all(g_sel == o_sel, axis=-1)  # [B][Hkv]
        differ += int(bad.sum())
        if bad.any():
            tie_b = {(b, g) for b in range(w.B) for g in range(w.Hkv)
                     if near_tie_units(W[b:b + 1, g:g + 1], lens[b:b + 1], w.S, w.k)}
            differ_outside += sum(1 for b, g in zip(*np.nonzero(bad)) if (b, g) not in tie_b)
            h = host[li]
            o_out = oracle.sparse_attn(OL, h["q"], h["k_pool"], h["v_pool"], h["k_scales"], h["v_scales"],
                                       h["table"], lens, g_sel, sm)  # attention on the GPU's selection
        d = g_out.astype(np.float64) - o_out
        err = max(err, float(np.abs(d).max()))
        num += float((d * d).sum())
        den += float((o_out * o_out).sum())
    parity = {"layer_steps": n_steps, "units": n_steps * units, "near_tie_units": ties,
              "selection_units_differing": differ, "selection_units_differing_outside_near_ties": differ_outside,
              "attention_max_abs_err": err, "attention_rel_l2": math.sqrt(num / den) if den > 0 else 0.0,
              "bars": {"selection": "bit-exact outside near ties (1e-4 relative)", "max_abs_err": 1e-2,
                       "rel_l2": 5e-3}}
    info = host_info()
    baseline = {"value": round(w.B * n_steps / dtn, 3), "unit": "query-tokens/s/layer", "cores": threads,
                "kind": "oracle",
                "sample": f"{n_steps} full layer-step(s) of {w.name} (all {w.B} sequences, {units} units: "
                          f"append, bounds, selection, attention), fp64, the (sequence, KV head) units "
                          f"fanned out over {threads} threads: {dtn:.2f} s; one thread: {dt1:.2f} s",
                "single_thread_value": round(w.B * n_steps / dt1, 3), **info}
    return baseline, parity


if __name__ == "__main__":
    sys.exit(main())
