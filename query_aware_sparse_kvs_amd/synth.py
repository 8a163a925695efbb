"""Seeded synthetic decode workloads.

This module only draws inputs: queries, paged K/V pools, block tables,
sequence lengths, fp8 codes with their group scales, and the drifting
selections of the hot-buffer workload.  It computes none of the method's
arithmetic (no summaries, bounds, selection or attention), so the HIP path
and the CPU oracle can both be fed from it.

Shapes of the five workloads, with the reading of each recipe:

* ``tiny``      1 sequence, 4 query / 2 KV heads, head dim 64, 1024 tokens in
                16-token blocks, k = 8; fp32 N(0,1); identity block table.
* ``llama8b``   8 sequences, 32 / 4 heads, head dim 128, 32768 tokens in
                64-token blocks (512), k = 128; bf16 N(0,1); 2 % of the tokens
                of every (sequence, KV head) replaced by 4*sqrt(d)*u with u a
                random unit vector of that (layer, sequence, KV head);
                pages randomly permuted; 32 layer instances.
* ``highconc``  256 sequences, same heads, 32768 tokens, k = 32; the 655
                planted tokens of a (sequence, KV head) sit inside 26 (5 %)
                random blocks; one shared pool of 131072 shuffled pages.
* ``hotbuf``    the ``llama8b`` data with 128 hot slots per (sequence, KV
                head) and a selection that drifts by 13 (10 % of 128) blocks a
                step.
* ``longfp8``   4 sequences, 131072 tokens (2048 blocks), k = 64; K/V drawn
                N(0,1) with one outlier channel per KV head (ceil(0.5 % of
                128)) scaled x8, then stored as OCP E4M3FN codes with one fp32
                scale per 32 channels of a token (scale = absmax / 448, 1 for
                an all-zero group; round to nearest even, saturated); bf16 q;
                16 layer instances (a step reads only 48 MiB, so fewer would
                fit in the 256 MB last-level cache).

The pages speak of large models (an 8B model with 32 layers, 4 KV heads and
head dim 128; GLM-5.1-FP8 at 32K+8K tokens and 256 requests).  Their weights
and prompts are not used: these random tensors of the same shapes stand in.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    L: int
    k: int
    q_dtype: str            # "f32" | "bf16"
    kv_dtype: str           # "f32" | "bf16" | "e4m3"
    quant_group: int = 0
    layers: int = 1
    heavy: str = "none"     # "none" | "scattered" | "clustered"
    heavy_frac: float = 0.0
    heavy_scale: float = 4.0
    heavy_block_frac: float = 0.0
    table: str = "permuted"  # "identity" | "permuted"
    hot_slots: int = 0
    drift: int = 0
    outlier_channels: int = 0
    outlier_mult: float = 1.0
    seed: int = 0

    @property
    def nb(self) -> int:
        return (self.L + self.S - 1) // self.S

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    "tiny": Workload("tiny", B=1, Hq=4, Hkv=2, D=64, S=16, L=1024, k=8, q_dtype="f32",
                     kv_dtype="f32", table="identity", seed=1),
    "llama8b": Workload("llama8b", B=8, Hq=32, Hkv=4, D=128, S=64, L=32768, k=128,
                        q_dtype="bf16", kv_dtype="bf16", layers=32, heavy="scattered",
                        heavy_frac=0.02, heavy_scale=4.0, seed=2),
    "highconc": Workload("highconc", B=256, Hq=32, Hkv=4, D=128, S=64, L=32768, k=32,
                         q_dtype="bf16", kv_dtype="bf16", heavy="clustered", heavy_frac=0.02,
                         heavy_scale=4.0, heavy_block_frac=0.05, seed=3),
    "hotbuf": Workload("hotbuf", B=8, Hq=32, Hkv=4, D=128, S=64, L=32768, k=128,
                       q_dtype="bf16", kv_dtype="bf16", layers=32, heavy="scattered",
                       heavy_frac=0.02, heavy_scale=4.0, hot_slots=128, drift=13, seed=4),
    "longfp8": Workload("longfp8", B=4, Hq=32, Hkv=4, D=128, S=64, L=131072, k=64,
                        q_dtype="bf16", kv_dtype="e4m3", quant_group=32, layers=16,
                        outlier_channels=1, outlier_mult=8.0, seed=5),
}

# order of the workloads as numbered in the benchmark configuration list
WORKLOAD_ORDER = ["tiny", "llama8b", "highconc", "hotbuf", "longfp8"]

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
E4M3_MAX = 448.0


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields changed (smaller test shapes)."""
    return replace(w, **kw)


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _randn(shape, dtype, device, gen):
    return torch.randn(shape, dtype=dtype, device=device, generator=gen)


def block_table(w: Workload, device, layer: int = 0, max_blocks: int | None = None,
                num_pages: int | None = None) -> torch.Tensor:
    """[B][max_blocks] int32 page ids; logical blocks beyond nb are -1."""
    max_blocks = w.nb if max_blocks is None else max_blocks
    used = w.B * w.nb
    num_pages = used if num_pages is None else num_pages
    assert num_pages >= used and max_blocks >= w.nb
    if w.table == "identity":
        pages = torch.arange(used, device=device, dtype=torch.int64)
    else:
        g = _gen(device, w.seed, 100 + layer)
        pages = torch.randperm(num_pages, device=device, generator=g)[:used]
    tbl = torch.full((w.B, max_blocks), -1, dtype=torch.int32, device=device)
    tbl[:, : w.nb] = pages.view(w.B, w.nb).to(torch.int32)
    return tbl


def _plant_heavy(w: Workload, pool: torch.Tensor, table: torch.Tensor, layer: int,
                 stream: int) -> None:
    """Replaces heavy_frac of every (sequence, KV head)'s tokens by
    heavy_scale*sqrt(D)*u, u a random unit vector of that unit."""
    if w.heavy == "none" or w.heavy_frac <= 0:
        return
    device = pool.device
    g = _gen(device, w.seed, stream + layer)
    n_heavy = int(round(w.heavy_frac * w.L))
    for b in range(w.B):
        for h in range(w.Hkv):
            u = torch.randn(w.D, generator=g, device=device, dtype=torch.float32)
            u = u / u.norm()
            vec = (w.heavy_scale * math.sqrt(w.D)) * u
            if w.heavy == "scattered":
                toks = torch.randperm(w.L, generator=g, device=device)[:n_heavy]
            else:
                n_blk = max(1, int(round(w.heavy_block_frac * w.nb)))
                blks = torch.randperm(w.nb, generator=g, device=device)[:n_blk]
                slots = (blks[:, None] * w.S + torch.arange(w.S, device=device)[None, :]).reshape(-1)
                slots = slots[slots < w.L]
                take = min(n_heavy, slots.numel())
                toks = slots[torch.randperm(slots.numel(), generator=g, device=device)[:take]]
            pages = table[b, toks // w.S].long()
            pool[pages, h, toks % w.S, :] = vec.to(pool.dtype)


def quantize_e4m3(x: torch.Tensor, group: int):
    """Harness-side cache write of fp8 K/V: per (token, 32-channel group)
    symmetric scale absmax/448 (1 for an all-zero group), codes rounded to
    nearest even by torch's float8_e4m3fn cast after clamping to +-448.
    Returns (codes uint8 with x's shape, scales fp32 [..., D/group])."""
    D = x.shape[-1]
    xg = x.float().reshape(*x.shape[:-1], D // group, group)
    absmax = xg.abs().amax(dim=-1)
    scale = torch.where(absmax > 0, absmax / E4M3_MAX, torch.ones_like(absmax))
    y = (xg / scale[..., None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(x.shape)
    return codes.contiguous(), scale.contiguous()


def v_pool_shape(P: int, Hkv: int, D: int, S: int) -> tuple:
    """Shape of a V pool: each tile is cut into runs of T = min(S, 32)
    consecutive tokens, each stored channel-major."""
    T = min(S, 32)
    return (P, Hkv, S // T, D, T)


def v_tiles_from_token_major(x: torch.Tensor) -> torch.Tensor:
    """[..., S, D] token-major tiles -> the V pool layout [..., S/T, D, T]."""
    S, D = x.shape[-2], x.shape[-1]
    T = min(S, 32)
    return x.reshape(*x.shape[:-2], S // T, T, D).transpose(-1, -2).contiguous()


def make_inputs(w: Workload, device="cpu", layer: int = 0, seq_lens=None,
                max_blocks: int | None = None, num_pages: int | None = None) -> dict:
    """All inputs of one decode layer-step.

    Returns a dict with q [B][Hq][D], k_pool [P][Hkv][S][D] and v_pool
    [P][Hkv][S/T][D][T], T = min(S, 32) (V tiles as runs of T tokens, each
    channel-major; fp32, bf16 or uint8 E4M3FN codes), k_scales / v_scales
    [P][Hkv][S][D/group] fp32 (fp8 only, else None), block_table
    [B][max_blocks] int32, seq_lens [B] int32.  Token positions at or past a
    sequence's length still hold random data (they must not be read)."""
    device = torch.device(device)
    mb = w.nb if max_blocks is None else max_blocks
    tbl = block_table(w, device, layer, mb, num_pages)
    P = w.B * w.nb if num_pages is None else num_pages
    shape = (P, w.Hkv, w.S, w.D)
    base = 1000 * (layer + 1)
    q = _randn((w.B, w.Hq, w.D), _TORCH_DT[w.q_dtype], device, _gen(device, w.seed, base + 1))
    out = {"q": q, "block_table": tbl}
    if w.kv_dtype in ("f32", "bf16"):
        dt = _TORCH_DT[w.kv_dtype]
        kp = _randn(shape, dt, device, _gen(device, w.seed, base + 2))
        vp = _randn(v_pool_shape(P, w.Hkv, w.D, w.S), dt, device, _gen(device, w.seed, base + 3))
        _plant_heavy(w, kp, tbl, layer, 10_000)
        out.update(k_pool=kp, v_pool=vp, k_scales=None, v_scales=None)
    else:
        assert w.kv_dtype == "e4m3" and w.quant_group > 0
        for name, stream in (("k", 2), ("v", 3)):
            x = _randn(shape, torch.float32, device, _gen(device, w.seed, base + stream))
            if w.outlier_channels > 0:
                g = _gen(device, w.seed, base + 10 + stream)
                for h in range(w.Hkv):
                    ch = torch.randperm(w.D, generator=g, device=device)[: w.outlier_channels]
                    x[:, h, :, ch] *= w.outlier_mult
            if name == "k":
                _plant_heavy(w, x, tbl, layer, 10_000)
            codes, scales = quantize_e4m3(x, w.quant_group)
            del x
            if name == "v":  # token-major [S][D] -> runs of T tokens, channel-major
                codes = v_tiles_from_token_major(codes)
            out[name + "_pool"] = codes
            out[name + "_scales"] = scales
    if seq_lens is None:
        seq_lens = torch.full((w.B,), w.L, dtype=torch.int32, device=device)
    else:
        seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32, device=device)
    out["seq_lens"] = seq_lens
    return out


def newest_tokens(w: Workload, inp: dict) -> dict:
    """The K/V elements (and fp8 scales) each sequence holds at its last
    position seq_lens[b]-1, gathered from the pools as [B][Hkv][D] (scales
    [B][Hkv][D/group]): a decode token that, appended again, leaves the cache
    as it is."""
    lens = inp["seq_lens"].long()
    t = (lens - 1).clamp(min=0)
    pages = inp["block_table"].long().gather(1, (t // w.S)[:, None])[:, 0]
    s = t % w.S
    T = min(w.S, 32)
    out = {"k_new": inp["k_pool"][pages, :, s, :].contiguous(),
           "v_new": inp["v_pool"][pages, :, s // T, :, s % T].contiguous()}
    for n in ("k", "v"):
        sc = inp[n + "_scales"]
        out[n + "_new_scales"] = None if sc is None else sc[pages, :, s, :].contiguous()
    return out


def random_selection(w: Workload, seq_lens, k: int, seed: int, max_fill: bool = True) -> np.ndarray:
    """A valid selection [B][Hkv][k] (ascending ids then -1), drawn at random
    for attention-only tests: sink and newest block included, the rest a
    uniform subset of the middle blocks."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens)
    sel = np.full((len(seq_lens), w.Hkv, k), -1, dtype=np.int32)
    for b, L in enumerate(seq_lens):
        nb = (int(L) + w.S - 1) // w.S
        for h in range(w.Hkv):
            if nb <= k:
                ids = np.arange(nb)
            else:
                n_mid = k - 2 if max_fill else int(rng.integers(0, k - 1))
                mid = rng.choice(np.arange(1, nb - 1), size=n_mid, replace=False)
                ids = np.sort(np.concatenate([[0, nb - 1], mid]))
            sel[b, h, : len(ids)] = ids
    return sel


def drift_selections(sel0: np.ndarray, nb: int, steps: int, drift: int, seed: int) -> np.ndarray:
    """Hot-buffer selection stream: returns [steps+1][B][Hkv][k] where entry 0
    is sel0 and each later step swaps `drift` non-forced members of the
    previous set for `drift` blocks outside it (blocks 0 and nb-1 are never
    swapped), both drawn uniformly from one seeded stream; rows stay sorted."""
    rng = np.random.default_rng(seed)
    B, H, k = sel0.shape
    out = np.empty((steps + 1, B, H, k), dtype=np.int32)
    out[0] = sel0
    for t in range(1, steps + 1):
        for b in range(B):
            for h in range(H):
                prev = out[t - 1, b, h]
                cur = prev[prev >= 0]
                movable = cur[(cur != 0) & (cur != nb - 1)]
                outside = np.setdiff1d(np.arange(1, nb - 1), cur, assume_unique=False)
                n = min(drift, movable.size, outside.size)
                drop = rng.choice(movable, size=n, replace=False)
                add = rng.choice(outside, size=n, replace=False)
                new = np.sort(np.concatenate([np.setdiff1d(cur, drop), add]))
                row = np.full(k, -1, dtype=np.int32)
                row[: new.size] = new
                out[t, b, h] = row
    return out
