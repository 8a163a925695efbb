"""A decode layer-step captured into a HIP graph gives, on every replay, the
same results as the eager calls (the path records no memset nodes; this
checks it with replays separated by unrelated eager work), also when the
batch runs as concurrent slices on several streams (fork and join inside the
graph), which must give bit-identical results to the one-chain step."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("parts", [1, 3])
def test_graph_replays_match_eager(orc, parts):
    import torch
    from query_aware_sparse_kvs_amd import kvs, synth
    from query_aware_sparse_kvs_amd.step import SparseDecodeStep

    dev = torch.device("cuda:0")
    w = synth.scaled(synth.WORKLOADS["llama8b"], B=4, L=9000, k=24, layers=1)
    inp = synth.make_inputs(w, dev, seq_lens=[9000, 8191, 64, 4000])
    code = kvs.DTYPE_CODE
    L = kvs.Layout(w.B, w.Hq, w.Hkv, w.D, w.S, w.nb, w.B * w.nb, code[w.q_dtype], code[w.kv_dtype])
    st = SparseDecodeStep(L, w.k, dev, parts=parts)
    assert len(st.slices) == parts
    summ = st.new_summaries(dev)
    st.prefill_summaries(inp["k_pool"], None, inp["block_table"], inp["seq_lens"], summ)

    def step():
        return st.run(inp["q"], inp["k_pool"], inp["v_pool"], None, None, inp["block_table"],
                      inp["seq_lens"], summ)

    eager_out = step().clone()
    eager_sel = st.sel.clone()
    torch.cuda.synchronize()
    if parts > 1:  # the same kernels on the same rows: bit-identical to one chain
        one = SparseDecodeStep(L, w.k, dev, parts=1)
        one.run(inp["q"], inp["k_pool"], inp["v_pool"], None, None, inp["block_table"], inp["seq_lens"],
                summ)
        torch.cuda.synchronize()
        assert torch.equal(one.sel, eager_sel) and torch.equal(one.out, eager_out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        st.out.fill_(float("nan"))
        st.sel.fill_(-9)
        junk = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.sel, eager_sel), f"replay {rep}: selection differs"
        assert torch.equal(st.out, eager_out), f"replay {rep}: output differs"
        del junk
    assert kvs.kvs_device_errors() == 0


@pytest.mark.parametrize("route", ["fused", "separate"])
def test_decode_step_with_append_graph_replays_match_eager(orc, route):
    """The whole decode step as the benchmark replays it -- the decode token
    appended again at its own position (the cache does not change), scores,
    and the top-k inside the attention launch (or as a launch of its own) --
    captured into a graph gives the eager selection and output on every
    replay, with unrelated eager work between replays."""
    import torch
    from query_aware_sparse_kvs_amd import kvs, synth
    from query_aware_sparse_kvs_amd.step import SparseDecodeStep

    dev = torch.device("cuda:0")
    w = synth.scaled(synth.WORKLOADS["llama8b"], B=4, L=9000, k=24, layers=1)
    inp = synth.make_inputs(w, dev, seq_lens=[9000, 8191, 64, 4001])
    code = kvs.DTYPE_CODE
    L = kvs.Layout(w.B, w.Hq, w.Hkv, w.D, w.S, w.nb, w.B * w.nb, code[w.q_dtype], code[w.kv_dtype])
    st = SparseDecodeStep(L, w.k, dev)
    summ = st.new_summaries(dev)
    st.prefill_summaries(inp["k_pool"], None, inp["block_table"], inp["seq_lens"], summ)
    nt = synth.newest_tokens(w, inp)
    tok = kvs.AppendArgs(k_new=nt["k_new"], v_new=nt["v_new"], k_new_scales=None, v_new_scales=None,
                         block_table=inp["block_table"], k_pool=inp["k_pool"], v_pool=inp["v_pool"])
    run = st.run_decode_fused if route == "fused" else st.run_decode

    def step():
        return run(inp["q"], tok, inp["seq_lens"], summ)

    eager_out = step().clone()
    eager_sel = st.sel.clone()
    eager_summ = summ.clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        st.out.fill_(float("nan"))
        st.sel.fill_(-9)
        junk = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.sel, eager_sel), f"replay {rep}: selection differs"
        assert torch.equal(st.out, eager_out), f"replay {rep}: output differs"
        # bit patterns: blocks past a sequence's end hold whatever the
        # allocation held, NaN patterns included
        assert torch.equal(summ.view(torch.int16), eager_summ.view(torch.int16)), f"replay {rep}: summaries changed"
        del junk
    assert kvs.kvs_device_errors() == 0
