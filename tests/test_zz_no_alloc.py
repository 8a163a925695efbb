"""kvs_sparse_decode_attn_noalloc (split partials in the library's device
array instead of a caller's workspace) against kvs_sparse_decode_attn on the
same inputs, through the C ABI: bit-identical outputs (same kernels, same
splits), both within the oracle's attention bars.  Two calls in a row, the
second on a smaller input, so the array holds the first call's partials when
the second runs; an fp8 layout and a single-split layout (partials unused)
as well."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ATOL, RTOL_L2 = 1e-2, 5e-3
REG_ATOL, REG_RTOL_L2 = 3e-4, 5e-5  # regression bars (test_gpu_parity.py states their basis)


def _np(t):
    import torch
    t = t.cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _case(orc, torch, kvs, synth, dev, base, over, lens, k, seed_sel):
    w = synth.scaled(synth.WORKLOADS[base], **over, k=k)
    inp = synth.make_inputs(w, dev, seq_lens=lens)
    code = kvs.DTYPE_CODE
    P = inp["k_pool"].shape[0]
    L = kvs.Layout(w.B, w.Hq, w.Hkv, w.D, w.S, w.nb, P, code[w.q_dtype], code[w.kv_dtype], w.quant_group)
    h_lens = inp["seq_lens"].cpu().numpy()
    sel = synth.random_selection(w, h_lens, k, seed=seed_sel)
    sel_d = torch.from_numpy(sel).to(dev)
    sm = 1.0 / math.sqrt(w.D)
    ws = torch.zeros(kvs.kvs_attn_workspace_size(L, k), dtype=torch.uint8, device=dev)
    ref = torch.full((w.B, w.Hq, w.D), float("nan"), device=dev)
    kvs.kvs_sparse_decode_attn(L, kvs.KVS_TABLE_PAGED, inp["q"], inp["k_pool"], inp["v_pool"], inp["k_scales"],
                               inp["v_scales"], inp["block_table"], inp["seq_lens"], sel_d, k, sm, ref, ws)
    out = torch.full_like(ref, float("nan"))
    kvs.kvs_sparse_decode_attn_noalloc(L, kvs.KVS_TABLE_PAGED, inp["q"], inp["k_pool"], inp["v_pool"],
                                       inp["k_scales"], inp["v_scales"], inp["block_table"], inp["seq_lens"],
                                       sel_d, k, sm, out)
    torch.cuda.synchronize()
    assert kvs.kvs_device_errors(clear=True) == 0
    OL = orc.Layout(w.B, w.Hq, w.Hkv, w.D, w.S, w.nb, P, code[w.kv_dtype], w.quant_group)
    sc = lambda n: None if inp[n] is None else inp[n].cpu().numpy()
    o = orc.sparse_attn(OL, inp["q"].double().cpu().numpy(), _np(inp["k_pool"]), _np(inp["v_pool"]),
                        sc("k_scales"), sc("v_scales"), inp["block_table"].cpu().numpy(), h_lens, sel, sm)
    g = out.double().cpu().numpy()
    assert np.isfinite(g).all()
    err = np.abs(g - o).max()
    rel = np.linalg.norm(g - o) / np.linalg.norm(o)
    assert err <= ATOL and rel <= RTOL_L2, f"max|err| {err:.3e}, rel L2 {rel:.3e}"
    assert err <= REG_ATOL and rel <= REG_RTOL_L2, "regression bar: " + f"max|err| {err:.3e}, rel L2 {rel:.3e}"
    assert torch.equal(out, ref), "no-allocation attention differs from the workspace entry point"
    return kvs.kvs_attn_num_splits(L, k), err, rel


def test_noalloc_attention_matches_workspace_entry_point(orc):
    import torch
    from query_aware_sparse_kvs_amd import kvs, synth
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kvs.kvs_device_errors(clear=True)
    cases = [
        # the larger call first, then a smaller one (fewer rows and splits)
        ("bf16-large", "llama8b", {"B": 4, "L": 9000, "layers": 1}, [9000, 8191, 4097, 65], 32, 1),
        ("bf16-small", "llama8b", {"B": 2, "L": 3000, "layers": 1}, [3000, 1001], 9, 2),
        ("fp8", "longfp8", {"B": 2, "L": 6000}, [6000, 2049], 16, 3),
        ("bf16-one-split", "llama8b", {"B": 64, "L": 640, "layers": 1}, None, 4, 4),
    ]
    for name, base, over, lens, k, seed in cases:
        print(f"[noalloc {name}] k={k} lens={lens}", flush=True)
        n, err, rel = _case(orc, torch, kvs, synth, dev, base, over, lens, k, seed)
        print(f"[noalloc {name}] splits {n}: identical; max|err| {err:.2e} rel L2 {rel:.2e}", flush=True)
