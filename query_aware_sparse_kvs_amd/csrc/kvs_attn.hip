// kvs_attn.hip -- attention over the selected blocks only (page "KV 稀疏化",
// §5 "Quest", last step), tiled with a running max and normaliser per tile
// that are merged across tiles and splits ("分块稀疏注意力与KV Cache量化…",
// §2.2), fp8 K/V dequantised inside the read (same page, §1.3).
//
// Work split (both kernels): a (sequence, KV head) unit's k selected blocks
// are cut into `nsplit` runs of `bps` entries; one 256-thread workgroup
// (4 wavefronts) handles one run, each wavefront one tile at a time (the
// MFMA kernels' tiles are 32-token halves of 64-token blocks, or whole
// 32-token blocks; the VALU kernel's tiles are whole blocks).
// The four wavefronts' running (max, sum, acc) are merged in LDS and written
// as a split partial (or, with a single split, as the output row);
// merge_kernel then merges the splits of every query head:
//   m* = max m_i, l* = sum l_i 2^(m_i-m*), o = sum acc_i 2^(m_i-m*) / l*.
// (The merge needs the partials of workgroups on other XCDs, whose L2
// caches are not coherent within a kernel; a kernel boundary is far cheaper
// than a device-scope release per workgroup.)
// Scores are kept in base 2: the query is scaled by sm_scale*log2(e).
//
// attn_mfma_kernel (bf16, blocks of 32 or 64 tokens): both products run on
// v_mfma_f32_16x16x32_bf16 with the G query heads padded to 16 columns.
//   scores  S^T = K Q^T: the A operand is 16 token rows x 32 channels of K,
//           loaded straight from the token-major tile with 16-byte loads;
//           B is Q^T, loaded once.  Token rows are permuted (tau below) so
//           that the accumulator a lane ends up holding is exactly the
//           8-token slice it must feed to the value product.
//   values  O^T = V^T P^T: the A operand is 16 channels x 32 tokens of one
//           32-token run of the V tile, stored channel-major, so each load
//           instruction reads 1 KiB contiguous; B is P^T taken
//           from the score accumulators in registers.  P is split into
//           hi = bf16(p) and lo = bf16(p - hi), two MFMAs, so the product
//           keeps ~16 bits of P.  No LDS traffic inside the tile loop.
//   A wavefront resolves its tiles (selection -> table) for all of them at
//   once into LDS, then streams them through a two-stage software pipeline:
//   the next tile's K is requested as soon as the current tile's scores are
//   computed, its V as soon as the current value product is, so about one
//   tile (16 KiB of K and V at d = 128) stays in flight per wavefront.
// attn_valu_kernel (fp32, fp8, and bf16 with S = 16): lane = token for the
//   scores (64/S lanes split a token's channels), lane = channel pair for the
//   values, probabilities broadcast through LDS; every K/V load of a tile is
//   issued before any of its arithmetic.
// Roofline: HBM-bound gather of 2*S*D*elem bytes (+ fp8 scales) per
// selected block.
#include <type_traits>

#include "kvs_append.h"
#include "kvs_internal.h"
#include "kvs_topk.h"

namespace kvs {
namespace {

constexpr int kGMax = 16;
constexpr int kAttnWaves = 4;  // wavefronts per workgroup of the MFMA kernels
// tokens per tile of the MFMA kernels: a 64-token cache block is streamed as
// its two 32-token halves (the K rows and the V runs of a half are
// contiguous in the block's tiles), which keeps more of a wavefront's work
// behind its loads than whole 64-token pages
constexpr int kAttnTile = 32;
constexpr int kComputeUnits = 256;  // MI355X

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// A wavefront-uniform 64-bit value held in scalar registers.
__device__ __forceinline__ long long uniform64(long long v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(unsigned)(unsigned long long)v);
  const int hi = __builtin_amdgcn_readfirstlane((int)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Reads an input that no kernel of the call writes, at a wavefront-uniform
// address, through the constant address space: the compiler then issues a
// scalar load, which does not wait behind vector loads in flight.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Shared entry checks of one selection slot.  Returns the tile's pool entry
// (page or hot slot), or -1 when the slot is padding or invalid.
__device__ __forceinline__ int tile_entry(const AttnArgs& a, const int32_t* srow, int i, int b, int g,
                                          int nb, int lane, int* j_out) {
  const int j = ld_uniform(srow + i);
  if (j < 0) {
    if (j != -1 && lane == 0) raise_flag(a.err, 0x4u);
    return -1;
  }
  const int jp = i > 0 ? ld_uniform(srow + i - 1) : -1;
  if (j >= nb || (i > 0 && (jp >= j || jp < 0))) {
    if (lane == 0) raise_flag(a.err, 0x4u);
    if (j >= nb) return -1;
  }
  const int entry = a.hot ? ld_uniform(a.table + ((long long)b * a.Hkv + g) * a.MB + j)
                          : ld_uniform(a.table + (long long)b * a.MB + j);
  if (entry < 0 || entry >= a.P) {
    if (lane == 0) raise_flag(a.err, 0x2u);
    return -1;
  }
  *j_out = j;
  return entry;
}

// The work index of workgroup w of n.  The dispatcher hands workgroups to
// the eight XCDs in turn (workgroup w, counted x-fastest, runs on XCD
// (w + s) % 8, s fixed for the launch: 0 launched alone, another value in a
// graph), and each XCD has its own L2; this numbering puts consecutive work
// indices on one XCD.  It is a permutation of 0..n-1 for any n (a tail of
// fewer than eight workgroups keeps its own numbers).
__device__ __forceinline__ int xcd_order(int w, int n) {
  const int per = n >> 3;  // workgroups per XCD in the whole rounds
  return w < 8 * per ? (w & 7) * per + (w >> 3) : w;
}

// The (split, KV head, sequence) a workgroup of a (nsplit, Hkv, B) grid
// works on, numbered by xcd_order: a unit's splits sit together on one XCD
// and share its scores, its table row and its query in one L2 instead of
// fetching them into eight.
__device__ __forceinline__ void xcd_unit(int& split, int& g, int& b) {
  const int nx = gridDim.x, ny = gridDim.y;
  const int m = xcd_order(blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z), nx * ny * gridDim.z);
  split = m % nx;
  const int u = m / nx;
  g = u % ny;
  b = u / ny;
}

__device__ __forceinline__ int clamp_len(const AttnArgs& a, int b, bool flag_it) {
  int len = ld_uniform(a.seq_lens + b);
  const int cap = a.MB * a.S;
  if (len < 0 || len > cap) {
    if (flag_it) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  return len;
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16)
// ---------------------------------------------------------------------------

// The K and V registers of one page in the MFMA layouts.  K: for each
// 32-token sub-tile h and row group tg, 16 token rows x 32 channels per
// k-step (A operand of the score product).  V: for each sub-tile, 16
// channels x 32 tokens per channel tile (A operand of the value product).
template <int D, int S>
struct PageK {
  u32x4 r[S / 32][2][D / 32];
};
template <int D, int S>
struct PageV {
  u32x4 r[S / 32][D / 16];
};

// kt: the page's K tile [S][D]; vt: its V tile [S/32][D][32] (32-token runs,
// each channel-major).
template <int D, int S>
__device__ __forceinline__ void load_page_k(const uint16_t* kt, int r, int j4, PageK<D, S>& K) {
#pragma unroll
  for (int h = 0; h < S / 32; ++h)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      // tau(tg, r): the token row lane-row r of group tg stands for
      const int row = h * 32 + 8 * (r >> 2) + 4 * tg + (r & 3);
#pragma unroll
      for (int cs = 0; cs < D / 32; ++cs)
        K.r[h][tg][cs] = *reinterpret_cast<const u32x4*>(kt + row * D + cs * 32 + 8 * j4);
    }
}
template <int D, int S>
__device__ __forceinline__ void load_page_v(const uint16_t* vt, int r, int j4, PageV<D, S>& V) {
#pragma unroll
  for (int h = 0; h < S / 32; ++h)
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
      V.r[h][ct] = *reinterpret_cast<const u32x4*>(vt + (h * D + ct * 16 + r) * 32 + 8 * j4);
}

// Scores of one page (ntok valid tokens, possibly 0), the online-softmax
// update of (m_run, l_run, o), and the P^T operands of the value product:
// lane (r, j4) holds tokens h*32 + 8*j4 + 4*tg + e of head r, which are
// exactly the 8 tokens it supplies to the value product of sub-tile h
// (slots 0..3 <- tg 0, 4..7 <- tg 1).  P = hi + lo, both bf16.
template <int D, int S>
__device__ __forceinline__ void page_scores(const PageK<D, S>& K, const bf16x8_t* qf, float q_scale, int ntok, int j4,
                                            float& m_run, float& l_run, f32x4_t* o, bf16x8_t* ph, bf16x8_t* pl) {
  constexpr int NSUB = S / 32, CS = D / 32, CT = D / 16;
  float s[NSUB][2][4];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int h = 0; h < NSUB; ++h)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cs = 0; cs < CS; ++cs)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(K.r[h][tg][cs]), qf[cs], sc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = h * 32 + 8 * j4 + 4 * tg + e;
        const float v = tok < ntok ? sc[e] * q_scale : -__builtin_inff();
        s[h][tg][e] = v;
        tmax = fmaxf(tmax, v);
      }
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = fmaxf(m_run, tmax);
  // nothing valid so far (m_new = -inf): leave everything as it is
  const float alpha = m_new == -__builtin_inff() ? 1.0f : exp2f(m_run - m_new);
  float psum = 0.0f;
#pragma unroll
  for (int h = 0; h < NSUB; ++h)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = s[h][tg][e];
        const float p = v == -__builtin_inff() ? 0.0f : exp2f(v - m_new);
        s[h][tg][e] = p;
        psum += p;
      }
  psum += __shfl_xor(psum, 16);
  psum += __shfl_xor(psum, 32);
  l_run = l_run * alpha + psum;
  m_run = m_new;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
#pragma unroll
  for (int h = 0; h < NSUB; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = e < 4 ? s[h][0][e] : s[h][1][e - 4];
      const __bf16 hb = static_cast<__bf16>(pv);
      ph[h][e] = hb;
      pl[h][e] = static_cast<__bf16>(pv - static_cast<float>(hb));
    }
}

// The value product of one page: o += V^T P^T, with V zeroed at token
// positions >= ntok (they may hold anything).
template <int D, int S>
__device__ __forceinline__ void page_values(PageV<D, S>& V, int ntok, int j4, const bf16x8_t* ph, const bf16x8_t* pl,
                                            f32x4_t* o) {
  constexpr int NSUB = S / 32, CT = D / 16;
#pragma unroll
  for (int h = 0; h < NSUB; ++h) {
    const int nt = ntok - h * 32;
    if (nt < 32) {
      const int t0 = 8 * j4;
      uint32_t keep[4];
#pragma unroll
      for (int w = 0; w < 4; ++w)
        keep[w] = (t0 + 2 * w < nt ? 0x0000FFFFu : 0u) | (t0 + 2 * w + 1 < nt ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int w = 0; w < 4; ++w) V.r[h][ct][w] &= keep[w];
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(V.r[h][ct]), ph[h], o[ct], 0, 0, 0);
      o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(V.r[h][ct]), pl[h], o[ct], 0, 0, 0);
    }
  }
}

// A wavefront's work list is over tiles of the selection: position i holds
// tile `i % sub` of selection slot i / sub (sub = tiles per cache block, 1
// or 2).  The position a lane resolves in chunk t0 of its wavefront's list
// is i = i0 + nw*(t0 + lane); it yields that slot's block j (-2 where there
// is no position), the block of the slot before it (jp; kFirstSlot for slot
// 0) and the tile's half of the block.
constexpr int kFirstSlot = -3;

__device__ __forceinline__ void fetch_slots(const int32_t* srow, int i0, int i1, int nw, int sub, int t0, int& j,
                                            int& jp, int& half) {
  const int lane = threadIdx.x & 63;
  const int i = i0 + nw * (t0 + lane);
  j = -2;  // no position
  jp = -1;
  half = 0;
  if (i < i1) {
    const int slot = sub == 2 ? i >> 1 : i;
    half = i - slot * sub;
    j = srow[slot];
    jp = slot > 0 ? srow[slot - 1] : kFirstSlot;
  }
}

// The unit's block-table row (paged: row b; hot: row (b, g)) copied into LDS
// by every thread of an NT-thread workgroup, when it has at most kTabMax
// entries; the caller synchronises the workgroup before reading it.
constexpr int kTabMax = 2048;

// In two halves, so that a kernel can issue the loads before it waits for
// anything else (the sequence length, say) and store them to LDS later.
template <int NT>
__device__ __forceinline__ void load_table_row(const AttnArgs& a, int b, int g, int (&v)[kTabMax / NT]) {
  const int32_t* row = a.hot ? a.table + ((long long)b * a.Hkv + g) * a.MB : a.table + (long long)b * a.MB;
#pragma unroll
  for (int x = 0; x < kTabMax / NT; ++x) {
    const int e = x * NT + (int)threadIdx.x;
    v[x] = e < a.MB ? row[e] : 0;
  }
}
template <int NT>
__device__ __forceinline__ void store_table_row(const AttnArgs& a, const int (&v)[kTabMax / NT], int* trow) {
#pragma unroll
  for (int x = 0; x < kTabMax / NT; ++x) {
    const int e = x * NT + (int)threadIdx.x;
    if (e < a.MB) trow[e] = v[x];
  }
}

// Resolves the chunk's positions (one per lane, from fetch_slots) into LDS:
// the index of the T-token tile in the pool (the cache's S-token blocks seen
// as sub = S/T consecutive tiles) and its valid token count (0 = nothing to
// do).  The table entry comes from the staged row `trow` when there is one,
// else from memory.
__device__ __forceinline__ void resolve_tiles(const AttnArgs& a, const int* trow, int j, int jp, int half, int b,
                                              int g, int nb, int len, int T, int sub, long long* wl_tile,
                                              int* wl_ntok) {
  const int lane = threadIdx.x & 63;
  long long tile = a.hot ? 0 : (long long)g * sub;  // the first tile of block (0, g): always in bounds
  int ntok = 0;
  if (j != -2) {
    bool ok = j >= 0;
    if (j < -1) raise_flag(a.err, 0x4u);
    if (ok) {
      if (j >= nb || (jp != kFirstSlot && (jp >= j || jp < 0))) raise_flag(a.err, 0x4u);
      ok = j < nb;
    }
    if (ok) {
      const int entry = trow ? trow[j]
                             : (a.hot ? a.table[((long long)b * a.Hkv + g) * a.MB + j] : a.table[(long long)b * a.MB + j]);
      if (entry < 0 || entry >= a.P) {
        raise_flag(a.err, 0x2u);
      } else {
        tile = (a.hot ? (long long)entry : (long long)entry * a.Hkv + g) * sub + half;
        ntok = max(0, min(T, len - j * a.S - half * T));
      }
    }
  }
  wl_tile[lane] = tile;
  wl_ntok[lane] = ntok;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Self-selecting mode: the workgroup picks its unit's blocks itself, from
// the scores, with the selection of kvs_topk.h (the same one topk_kernel
// runs), instead of reading a selection another launch wrote; the table
// row's loads go out beside the scores', both before the kernel waits for
// the sequence length.  self_select_finish returns the selection row (in
// LDS) after a workgroup barrier; the first split's workgroup also writes it
// to sel_out.
constexpr int kSelfSelMax = 2048;  // largest MB and k of the mode

// SELF: score ids per thread (0 = reads a selection): 2 up to 512 blocks,
// 8 up to kSelfSelMax
template <int NW, int SELF>
struct SelfSelLoads {
  double wv[SELF > 0 ? SELF : 1];  // the unit's scores, as load_unit_scores lays them out
  int tv[kTabMax / (64 * NW)];     // the table row, as load_table_row lays it out
};

template <int NW, int SELF>
__device__ __forceinline__ void self_select_load(const AttnArgs& a, int b, int g, bool staged,
                                                 SelfSelLoads<NW, SELF>& ld) {
  static_assert(NW * 64 == 256, "the selection runs on 256 threads");
  const long long unit = (long long)b * a.Hkv + g;
  load_unit_scores<SELF>(a.W + unit * a.MB, a.MB, ld.wv);
  if (staged) load_table_row<64 * NW>(a, b, g, ld.tv);
}

template <int NW, int SELF>
__device__ __forceinline__ const int32_t* self_select_finish(const AttnArgs& a, int b, int g, int split, int nb,
                                                             bool staged, const SelfSelLoads<NW, SELF>& ld,
                                                             int* trow, int32_t* lsel, TopkLds& tk) {
  const long long unit = (long long)b * a.Hkv + g;
  if (staged) store_table_row<64 * NW>(a, ld.tv, trow);
  select_unit<SELF>(ld.wv, a.MB, nb, a.k, a.recent, lsel, tk);
  __syncthreads();
  if (split == 0)
    for (int i = threadIdx.x; i < a.k; i += 64 * NW) a.sel_out[unit * a.k + i] = lsel[i];
  return lsel;
}

// The end of an MFMA-kernel workgroup: merges the NW wavefronts' running
// (max, sum, acc) in LDS; lane (r, j4) holds channels ct*16 + 4*j4 + e of
// head r.  Every wavefront stages its accumulator, then wavefront w merges
// channel tiles w*CT/NW .. (w+1)*CT/NW-1 of every head (the wavefronts'
// terms still added in order 0..NW-1).  One split: the normalised output
// row is written; otherwise the split partial.
template <int D, int NW>
__device__ __forceinline__ void wg_merge_write(const AttnArgs& a, int b, int g, int split, int wave, int r, int j4,
                                               float m_run, float l_run, const f32x4_t* o, float (*mg_m)[16],
                                               float (*mg_l)[16], float (*mg_o)[16][D + 4]) {
  constexpr int CT = D / 16;
  constexpr int CPW = CT / NW;  // channel tiles merged per wavefront
  static_assert(CT % NW == 0, "whole channel tiles per wavefront");
  const int G = a.G;
  if (j4 == 0) {
    mg_m[wave][r] = m_run;
    mg_l[wave][r] = l_run;
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    *reinterpret_cast<f32x4_t*>(&mg_o[wave][r][ct * 16 + 4 * j4]) = o[ct];
  __syncthreads();
  if (r >= G) return;
  float M = mg_m[0][r];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, mg_m[w][r]);
  float scw[NW], L = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float mw = mg_m[w][r];
    scw[w] = mw == -__builtin_inff() ? 0.0f : exp2f(mw - M);
    L += mg_l[w][r] * scw[w];
  }
  // one split: normalise and write the output row; else store the partial
  const bool direct = a.nsplit == 1;
  const float inv = direct ? (L > 0.0f ? 1.0f / L : 0.0f) : 1.0f;
  const long long hrow = (long long)b * a.Hq + (long long)g * G + r;
  const long long pi = hrow * a.nsplit + split;
  if (!direct && wave == 0 && j4 == 0) {
    a.part_m[pi] = M;
    a.part_l[pi] = L;
  }
  float* dst = direct ? a.out + hrow * D : a.part_acc + pi * D;
#pragma unroll
  for (int t = 0; t < CPW; ++t) {
    const int ct = wave * CPW + t;
    f32x4_t v[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) v[w] = *reinterpret_cast<const f32x4_t*>(&mg_o[w][r][ct * 16 + 4 * j4]);
    float4 res;
    float* pv = reinterpret_cast<float*>(&res);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = v[0][e] * scw[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) x += v[w][e] * scw[w];
      pv[e] = x * inv;
    }
    *reinterpret_cast<float4*>(dst + ct * 16 + 4 * j4) = res;
  }
}

// S: tokens per tile (kAttnTile); the cache's blocks hold a.S = S or 2S
// tokens, and a block of 2S tokens is streamed as its two tiles.
// The bf16 kernel's body.  TOK: the decode token is appended in the same
// launch (attn_mfma_tok_kernel, given selection, paged table): for the one
// tile that holds token len-1 its K row and V column come from the append
// arguments, whatever the pool still holds there, and each unit's first
// split workgroup writes the token into the cache (with its block's summary
// and the seal of a block it fills) after its own attention work.
template <int D, int S, int NW, int SELF, int TOK>
__device__ __forceinline__ void attn_mfma_body(const AttnArgs& a, const AppendArgs* ta) {
  static_assert(!TOK || (SELF == 0 && S == 32), "the token path streams 32-token tiles of a given selection");
  constexpr int CS = D / 32;  // k-steps of the score product
  constexpr int CT = D / 16;  // 16-channel tiles of the value product
  constexpr int NSUB = S / 32;  // 32-token sub-tiles per tile
  __shared__ float mg_m[NW][16], mg_l[NW][16];
  __shared__ float mg_o[NW][16][D + 4];
  __shared__ long long wl_tile[NW][64];
  __shared__ int wl_ntok[NW][64];
  __shared__ int trow[kTabMax];
  __shared__ int32_t lsel[SELF > 0 ? kSelfSelMax : 1];
  __shared__ TopkLds tk;
  __shared__ int wl_tok[TOK ? NW : 1][TOK ? 64 : 1];  // the token's row in the tile, or -1

  int split, g, b;
  xcd_unit(split, g, b);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j4 = lane >> 4;
  const int G = a.G;

  // B operand of the score product: Q^T, column r = query head g*G + r
  bf16x8_t qf[CS];
  {
    // columns past the group repeat its last head (their results are never
    // written): the loads are unconditional, so no wait for them is placed
    // before the loads that follow
    const int rq = min(r, G - 1);
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + ((long long)b * a.Hq + (long long)g * G + rq) * D;
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) qf[cs] = as_bf16x8(*reinterpret_cast<const uint4*>(qb + cs * 32 + 8 * j4));
  }
  // the token's K (this lane's 8 channels of every k-step) and V (channel
  // ct*16 + r of every channel tile), and the first split's append inputs
  u32x4 kn[TOK ? CS : 1];
  uint32_t vn[TOK ? CT : 1];
  TokenIn tin{0u, 0u, 1.0f, 0};
  if constexpr (TOK) {
    const long long unit = (long long)b * a.Hkv + g;
    const uint16_t* kb = static_cast<const uint16_t*>(ta->k_new) + unit * D;
    const uint16_t* vb = static_cast<const uint16_t*>(ta->v_new) + unit * D;
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) kn[cs] = *reinterpret_cast<const u32x4*>(kb + cs * 32 + 8 * j4);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) vn[ct] = vb[ct * 16 + r];
    tin = load_token_in<K_BF16, D, true>(*ta, b, g, split == 0, a.seq_lens);
  }
  const int sub = a.S / S;  // tiles per block: 1 or 2
  const int32_t* srow = a.sel + ((long long)b * a.Hkv + g) * a.k;  // self-selecting: replaced below
  // this split's selection slots, as tile positions; the wavefront's tiles
  // are positions i0, i0+NW, ...
  const int i0 = split * a.bps * sub + wave;
  const int i1 = min(split * a.bps + a.bps, a.k) * sub;
  const int ntiles = i0 < i1 ? (i1 - i0 + NW - 1) / NW : 0;
  // the loads that need no sequence length go out before it is awaited:
  // the unit's scores (self-selecting) or the first chunk's selection
  // slots, and the table row
  const bool staged = a.MB <= kTabMax;
  SelfSelLoads<NW, SELF> sl;
  int j0 = -2, jp0 = -1, h0 = 0;
  if constexpr (SELF > 0) {
    self_select_load<NW, SELF>(a, b, g, staged, sl);
  } else {
    fetch_slots(srow, i0, i1, NW, sub, 0, j0, jp0, h0);
    if (staged) load_table_row<64 * NW>(a, b, g, sl.tv);
  }
  const int len = clamp_len(a, b, tid == 0 && split == 0 && g == 0);
  const int nb = (len + a.S - 1) / a.S;  // blocks of the cache (a.S = S or 2S tokens)
  // the token: position len-1 (none for an empty sequence; a length past
  // the table was flagged and clamped, and appends nothing)
  const int raw_len = TOK ? ld_uniform(a.seq_lens + b) : 0;
  const bool tok_ok = TOK && raw_len >= 1 && raw_len <= a.MB * a.S;
  const int tok_t = tok_ok ? raw_len - 1 : -1;
  const int tok_j = tok_ok ? tok_t / a.S : -3, tok_half = tok_ok ? (tok_t % a.S) / S : 0;
  const int tok_row = tok_ok ? tok_t % S : -1;
  TokenBlock tblk{0, 0u, 0u};
  if constexpr (TOK) tblk = load_token_block<K_BF16, D, true, true>(*ta, b, g, raw_len, tok_ok && split == 0, a.seq_lens);

  float m_run = -__builtin_inff(), l_run = 0.0f;
  f32x4_t o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);

  // a software pipeline over the wavefront's tiles: K of the next tile is
  // requested as soon as this tile's scores are done, V as soon as its
  // value product is.  Every iteration issues the same loads, so the waits
  // stay exact; after the last page the request goes to the pool's first
  // tile of this KV head, which every workgroup of the head shares and the
  // caches keep (no HBM traffic)
  // the first chunk's slots and the table row are fetched together, so the
  // table lookups need no further round trip
  if constexpr (SELF > 0) {
    srow = self_select_finish<NW, SELF>(a, b, g, split, nb, staged, sl, trow, lsel, tk);
    fetch_slots(srow, i0, i1, NW, sub, 0, j0, jp0, h0);
  } else {
    if (staged) store_table_row<64 * NW>(a, sl.tv, trow);
    __syncthreads();
  }
  for (int t0 = 0; t0 < ntiles; t0 += 64) {  // chunks of 64 tiles
    int j = j0, jp = jp0, hf = h0;
    if (t0 > 0) fetch_slots(srow, i0, i1, NW, sub, t0, j, jp, hf);
    if constexpr (TOK) wl_tok[wave][lane] = j == tok_j && hf == tok_half ? tok_row : -1;  // (ordered by resolve)
    resolve_tiles(a, staged ? trow : nullptr, j, jp, hf, b, g, nb, len, S, sub, wl_tile[wave], wl_ntok[wave]);
    const int nt = min(64, ntiles - t0);
    PageK<D, S> K;
    PageV<D, S> V;
    {
      const long long tile = uniform64(wl_tile[wave][0]);
      load_page_k<D, S>(kpool + tile * S * D, r, j4, K);
      load_page_v<D, S>(vpool + tile * D * S, r, j4, V);
    }
    for (int tt = 0; tt < nt; ++tt) {
      const int ntok = __builtin_amdgcn_readfirstlane(wl_ntok[wave][tt]);
      const long long tnext = uniform64(tt + 1 < nt ? wl_tile[wave][tt + 1] : (a.hot ? 0 : (long long)g * sub));
      bf16x8_t ph[NSUB], pl[NSUB];
      int trw = -1;
      if constexpr (TOK) trw = __builtin_amdgcn_readfirstlane(wl_tok[wave][tt]);
      if (TOK && trw >= 0) {  // uniform: this tile holds the token; its K row from the arguments
#pragma unroll
        for (int tg = 0; tg < 2; ++tg)
          if (8 * (r >> 2) + 4 * tg + (r & 3) == trw)
#pragma unroll
            for (int cs = 0; cs < CS; ++cs) K.r[0][tg][cs] = kn[cs];
      }
      page_scores<D, S>(K, qf, a.q_scale, ntok, j4, m_run, l_run, o, ph, pl);
      load_page_k<D, S>(kpool + tnext * S * D, r, j4, K);
      if (TOK && trw >= 0 && (trw >> 3) == j4) {  // and its V column: element trw % 8 of this lane's run
        const int w = (trw & 7) >> 1;
        const bool hi = trw & 1;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          V.r[0][ct][w] = hi ? (V.r[0][ct][w] & 0x0000FFFFu) | (vn[ct] << 16) : (V.r[0][ct][w] & 0xFFFF0000u) | vn[ct];
      }
      page_values<D, S>(V, ntok, j4, ph, pl, o);
      load_page_v<D, S>(vpool + tnext * D * S, r, j4, V);
    }
  }

  wg_merge_write<D, NW>(a, b, g, split, wave, r, j4, m_run, l_run, o, mg_m, mg_l, mg_o);
  if constexpr (TOK) {
    // the unit's first split writes the token (this workgroup may have read
    // the token's tile: the seal reads it back past the L1)
    if (split == 0 && tok_ok) store_token<K_BF16, D, 64 * NW, true>(*ta, b, g, raw_len, tin, tblk);
  }
}

template <int D, int S, int NW, int SELF>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_mfma_kernel(AttnArgs a) {
  attn_mfma_body<D, S, NW, SELF, 0>(a, nullptr);
}

// attention over a given selection with the decode token appended in the
// same launch (bf16 K/V, paged table)
template <int D, int S, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_mfma_tok_kernel(AttnArgs a, AppendArgs t) {
  attn_mfma_body<D, S, NW, 0, 1>(a, &t);
}

// ---------------------------------------------------------------------------
// MFMA kernel for fp8 K/V (bf16 q)
// ---------------------------------------------------------------------------

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Eight fp8 codes -> eight floats (exact).
__device__ __forceinline__ void fp8x8_to_f32(u32x2 w, float* out) {
  fp8x4_to_f32(w.x, out);
  fp8x4_to_f32(w.y, out + 4);
}
// Eight E4M3FN codes -> bf16x8, exactly (every E4M3 value, subnormals
// included, is a bf16 value): gfx950's packed conversion with a unit scale,
// two codes per instruction.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(u32x2 w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
  return bf16x8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
// Eight floats -> hi = bf16(x), lo = bf16(x - hi): about 16 significant bits.
__device__ __forceinline__ void split_bf16(const float* f, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(f[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(f[e] - static_cast<float>(h));
  }
}

// K of one page: 8 codes of one token row per (sub-tile h, row group tg,
// k-step cs), in the A layout of the score product, and each one's scale.
template <int D, int S>
struct PageK8 {
  u32x2 k[S / 32][2][D / 32];
  float ks[S / 32][2][D / 32];
};
// V of one page: 8 codes (8 tokens of one channel) per (h, channel tile ct),
// in the A layout of the value product, and this lane's share of the page's
// V scales [S][groups] (at most 8 groups).
template <int D, int S>
struct PageV8 {
  u32x2 v[S / 32][D / 16];
  float vs[S * 8 / kWave];
};

template <int D, int S>
__device__ __forceinline__ void load_page_k8(const uint8_t* kt, const float* kst, int groups, const int* kgrp, int r,
                                             int j4, PageK8<D, S>& K) {
#pragma unroll
  for (int h = 0; h < S / 32; ++h)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      const int row = h * 32 + 8 * (r >> 2) + 4 * tg + (r & 3);  // tau(tg, r)
#pragma unroll
      for (int cs = 0; cs < D / 32; ++cs) {
        K.k[h][tg][cs] = *reinterpret_cast<const u32x2*>(kt + row * D + cs * 32 + 8 * j4);
        K.ks[h][tg][cs] = kst[row * groups + kgrp[cs]];
      }
    }
}
template <int D, int S>
__device__ __forceinline__ void load_page_v8(const uint8_t* vt, const float* vst, int groups, int r, int j4,
                                             int lane, PageV8<D, S>& V) {
#pragma unroll
  for (int h = 0; h < S / 32; ++h)
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
      V.v[h][ct] = *reinterpret_cast<const u32x2*>(vt + (h * D + ct * 16 + r) * 32 + 8 * j4);
#pragma unroll
  for (int y = 0; y < S * 8 / kWave; ++y) {
    const int x = y * kWave + lane;
    V.vs[y] = x < S * groups ? vst[x] : 0.0f;
  }
}

// K of one page for quantisation groups of 32 channels or more: the codes as
// in PageK8, and this lane's share of the page's K scales [S][groups] (as
// PageV8 holds the V scales), staged in LDS before the score product.
template <int D, int S>
struct PageK8G {
  u32x2 k[S / 32][2][D / 32];
  float ks[S * 8 / kWave];
};
template <int D, int S>
__device__ __forceinline__ void load_page_k8g(const uint8_t* kt, const float* kst, int groups, int r, int j4,
                                              int lane, PageK8G<D, S>& K) {
#pragma unroll
  for (int h = 0; h < S / 32; ++h)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      const int row = h * 32 + 8 * (r >> 2) + 4 * tg + (r & 3);  // tau(tg, r)
#pragma unroll
      for (int cs = 0; cs < D / 32; ++cs)
        K.k[h][tg][cs] = *reinterpret_cast<const u32x2*>(kt + row * D + cs * 32 + 8 * j4);
    }
#pragma unroll
  for (int y = 0; y < S * 8 / kWave; ++y) {
    const int x = y * kWave + lane;
    K.ks[y] = x < S * groups ? kst[x] : 0.0f;
  }
}

template <int D, int S>
__device__ __forceinline__ void page_softmax8(const float (*s)[2][4], float tmax, float& m_run, float& l_run,
                                              f32x4_t* o, float (*pf)[8]);

// Scores of one page.  K = fp32(decode(code) * scale) is split into two bf16
// (hi + lo) for the matrix product, so the scores keep ~16 bits of K.
// Returns the probabilities of this lane's 8 tokens per sub-tile (tokens
// h*32 + 8*j4 + e, the slots it supplies to the value product).
template <int D, int S>
__device__ __forceinline__ void page_scores8(const PageK8<D, S>& K, const bf16x8_t* qf, float q_scale, int ntok,
                                             int j4, float& m_run, float& l_run, f32x4_t* o, float (*pf)[8]) {
  constexpr int NSUB = S / 32, CS = D / 32;
  float s[NSUB][2][4];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int h = 0; h < NSUB; ++h)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        float x[8];
        fp8x8_to_f32(K.k[h][tg][cs], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= K.ks[h][tg][cs];
        bf16x8_t hi, lo;
        split_bf16(x, hi, lo);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, qf[cs], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, qf[cs], sc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = h * 32 + 8 * j4 + 4 * tg + e;
        const float v = tok < ntok ? sc[e] * q_scale : -__builtin_inff();
        s[h][tg][e] = v;
        tmax = fmaxf(tmax, v);
      }
    }
  page_softmax8<D, S>(s, tmax, m_run, l_run, o, pf);
}

// Online-softmax update of one page from its masked base-2 scores s (this
// lane's 8 tokens per sub-tile) and their lane-local maximum tmax: the new
// running max and normaliser, the rescaled accumulators, and the
// probabilities pf for the value product.
template <int D, int S>
__device__ __forceinline__ void page_softmax8(const float (*s)[2][4], float tmax, float& m_run, float& l_run,
                                              f32x4_t* o, float (*pf)[8]) {
  constexpr int NSUB = S / 32, CT = D / 16;
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = fmaxf(m_run, tmax);
  const float alpha = m_new == -__builtin_inff() ? 1.0f : exp2f(m_run - m_new);
  float psum = 0.0f;
#pragma unroll
  for (int h = 0; h < NSUB; ++h)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = s[h][tg][e];
        const float p = v == -__builtin_inff() ? 0.0f : exp2f(v - m_new);
        pf[h][4 * tg + e] = p;
        psum += p;
      }
  psum += __shfl_xor(psum, 16);
  psum += __shfl_xor(psum, 32);
  l_run = l_run * alpha + psum;
  m_run = m_new;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
}

// Scores of one page when every 32-channel k-step lies in one quantisation
// group: the codes decode exactly to bf16, one MFMA per k-step gives the
// group's partial dot product with q, and the token's group scale multiplies
// that fp32 partial (score = sum over groups of scale * (codes . q)).  Half
// the matrix products of page_scores8 and no hi/lo split; every product is
// exact and the sums are fp32.  ksl: this page's K scales in LDS as
// [group][S]; kgu[cs]: the group of k-step cs.
template <int D, int S>
__device__ __forceinline__ void page_scores8g(const PageK8G<D, S>& K, const bf16x8_t* qf, float q_scale, int ntok,
                                              int j4, const float* ksl, const int* kgu, float& m_run,
                                              float& l_run, f32x4_t* o, float (*pf)[8]) {
  constexpr int NSUB = S / 32, CS = D / 32;
  float s[NSUB][2][4];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int h = 0; h < NSUB; ++h)
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        const f32x4_t part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(K.k[h][tg][cs]), qf[cs],
                                                                     f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        // scales of this lane's 4 output tokens h*32 + 8*j4 + 4*tg + e
        const f32x4_t ks4 = *reinterpret_cast<const f32x4_t*>(ksl + kgu[cs] * S + h * 32 + 8 * j4 + 4 * tg);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = fmaf(part[e], ks4[e], sc[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = h * 32 + 8 * j4 + 4 * tg + e;
        const float v = tok < ntok ? sc[e] * q_scale : -__builtin_inff();
        s[h][tg][e] = v;
        tmax = fmaxf(tmax, v);
      }
    }
  page_softmax8<D, S>(s, tmax, m_run, l_run, o, pf);
}

// The value product of one page: V codes decode exactly to bf16; the V scale
// of (token, channel group) is folded into P per group (P' = p * scale,
// split hi + lo).  vsl: this page's V scales in LDS as [group][S].  Slots at
// or past ntok may hold any bytes, scales included (NaN, Inf): their P' is
// set to zero by selection, never by multiplying p = 0 with the scale.
template <int D, int S>
__device__ __forceinline__ void page_values8(const PageV8<D, S>& V, int ntok, int j4, const float (*pf)[8],
                                             const float* vsl, const int* ctgrp, f32x4_t* o) {
  constexpr int NSUB = S / 32, CT = D / 16;
#pragma unroll
  for (int h = 0; h < NSUB; ++h) {
    const int nt = ntok - h * 32;
    const int t0 = 8 * j4;
    // a sub-tile whose 32 slots all hold tokens needs no masks (uniform)
    const bool full = nt >= 32;
    uint32_t keep[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      keep[w] = (t0 + 2 * w < nt ? 0x0000FFFFu : 0u) | (t0 + 2 * w + 1 < nt ? 0xFFFF0000u : 0u);
    bf16x8_t phi, plo;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if (ct == 0 || ctgrp[ct] != ctgrp[ct - 1]) {  // uniform: a new channel group
        const float* vg = vsl + ctgrp[ct] * S + h * 32 + t0;
        const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(vg);
        const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(vg + 4);
        float pp[8];
        if (full) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pp[e] = pf[h][e] * s0[e];
            pp[4 + e] = pf[h][4 + e] * s1[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pp[e] = t0 + e < nt ? pf[h][e] * s0[e] : 0.0f;
            pp[4 + e] = t0 + 4 + e < nt ? pf[h][4 + e] * s1[e] : 0.0f;
          }
        }
        split_bf16(pp, phi, plo);
      }
      bf16x8_t a = fp8x8_to_bf16(V.v[h][ct]);
      if (!full) {  // positions past the sequence may hold anything
        u32x4 aw = __builtin_bit_cast(u32x4, a);
#pragma unroll
        for (int w = 0; w < 4; ++w) aw[w] &= keep[w];
        a = __builtin_bit_cast(bf16x8_t, aw);
      }
      o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, o[ct], 0, 0, 0);
      o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, o[ct], 0, 0, 0);
    }
  }
}

// PG: quantisation groups of 32 channels or more (page_scores8g), else the
// hi/lo score product (page_scores8).  S: tokens per tile, as in
// attn_mfma_kernel.
template <int D, int S, int NW, int SELF, int PG>
__global__ __launch_bounds__(64 * NW, 8 / NW) void attn_mfma8_kernel(AttnArgs a) {
  constexpr int CS = D / 32;
  constexpr int CT = D / 16;
  constexpr int NSUB = S / 32;
  __shared__ float mg_m[NW][16], mg_l[NW][16];
  __shared__ float mg_o[NW][16][D + 4];
  __shared__ long long wl_tile[NW][64];
  __shared__ int wl_ntok[NW][64];
  __shared__ int trow[kTabMax];
  __shared__ __attribute__((aligned(16))) float vsl[NW][S * 8];  // per wavefront: [group][S]
  __shared__ __attribute__((aligned(16))) float ksl[PG ? NW : 1][PG ? S * 8 : 1];  // K scales, same layout
  __shared__ int32_t lsel[SELF > 0 ? kSelfSelMax : 1];
  __shared__ TopkLds tk;

  int split, g, b;
  xcd_unit(split, g, b);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j4 = lane >> 4;
  const int G = a.G;
  const int groups = D / a.qg;  // 1, 2, 4 or 8 (qg >= 16)
  const int gshift = __builtin_ctz(groups);
  int kgrp[CS], ctgrp[CT];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs)
    kgrp[cs] = PG ? __builtin_amdgcn_readfirstlane((cs * 32) / a.qg) : (cs * 32 + 8 * j4) / a.qg;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) ctgrp[ct] = __builtin_amdgcn_readfirstlane((ct * 16) / a.qg);

  bf16x8_t qf[CS];  // B operand of the score product: Q^T, column r = query head g*G + r
  {
    const int rq = min(r, G - 1);  // (columns past the group repeat its last head, as in the bf16 kernel)
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + ((long long)b * a.Hq + (long long)g * G + rq) * D;
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) qf[cs] = as_bf16x8(*reinterpret_cast<const uint4*>(qb + cs * 32 + 8 * j4));
  }
  const int sub = a.S / S;  // tiles per block: 1 or 2
  const int32_t* srow = a.sel + ((long long)b * a.Hkv + g) * a.k;
  const int i0 = split * a.bps * sub + wave;  // tile positions, as in the bf16 kernel
  const int i1 = min(split * a.bps + a.bps, a.k) * sub;
  const int ntiles = i0 < i1 ? (i1 - i0 + NW - 1) / NW : 0;
  // the loads that need no sequence length first, as in the bf16 kernel
  const bool staged = a.MB <= kTabMax;
  SelfSelLoads<NW, SELF> sl;
  int j0 = -2, jp0 = -1, h0 = 0;
  if constexpr (SELF > 0) {
    self_select_load<NW, SELF>(a, b, g, staged, sl);
  } else {
    fetch_slots(srow, i0, i1, NW, sub, 0, j0, jp0, h0);
    if (staged) load_table_row<64 * NW>(a, b, g, sl.tv);
  }
  const int len = clamp_len(a, b, tid == 0 && split == 0 && g == 0);
  const int nb = (len + a.S - 1) / a.S;  // blocks of the cache (a.S = S or 2S tokens)

  float m_run = -__builtin_inff(), l_run = 0.0f;
  f32x4_t o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_pool);
  float* vw = vsl[wave];
  float* kw = ksl[PG ? wave : 0];

  // the same two-stage page pipeline as the bf16 kernel
  if constexpr (SELF > 0) {
    srow = self_select_finish<NW, SELF>(a, b, g, split, nb, staged, sl, trow, lsel, tk);
    fetch_slots(srow, i0, i1, NW, sub, 0, j0, jp0, h0);
  } else {
    if (staged) store_table_row<64 * NW>(a, sl.tv, trow);
    __syncthreads();
  }
  for (int t0 = 0; t0 < ntiles; t0 += 64) {
    int j = j0, jp = jp0, hf = h0;
    if (t0 > 0) fetch_slots(srow, i0, i1, NW, sub, t0, j, jp, hf);
    resolve_tiles(a, staged ? trow : nullptr, j, jp, hf, b, g, nb, len, S, sub, wl_tile[wave], wl_ntok[wave]);
    const int nt = min(64, ntiles - t0);
    typename std::conditional<PG != 0, PageK8G<D, S>, PageK8<D, S>>::type K;
    PageV8<D, S> V;
    {
      const long long tile = uniform64(wl_tile[wave][0]);
      if constexpr (PG)
        load_page_k8g<D, S>(kpool + tile * S * D, a.k_scales + tile * S * groups, groups, r, j4, lane, K);
      else
        load_page_k8<D, S>(kpool + tile * S * D, a.k_scales + tile * S * groups, groups, kgrp, r, j4, K);
      load_page_v8<D, S>(vpool + tile * D * S, a.v_scales + tile * S * groups, groups, r, j4, lane, V);
    }
    for (int tt = 0; tt < nt; ++tt) {
      const int ntok = __builtin_amdgcn_readfirstlane(wl_ntok[wave][tt]);
      const long long tnext = uniform64(tt + 1 < nt ? wl_tile[wave][tt + 1] : (a.hot ? 0 : (long long)g * sub));
      float pf[NSUB][8];
      if constexpr (PG) {
        // this page's K scales -> LDS as [group][S]
#pragma unroll
        for (int y = 0; y < S * 8 / kWave; ++y) {
          const int x = y * kWave + lane;
          if (x < S * groups) kw[(x & (groups - 1)) * S + (x >> gshift)] = K.ks[y];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        page_scores8g<D, S>(K, qf, a.q_scale, ntok, j4, kw, kgrp, m_run, l_run, o, pf);
        load_page_k8g<D, S>(kpool + tnext * S * D, a.k_scales + tnext * S * groups, groups, r, j4, lane, K);
      } else {
        page_scores8<D, S>(K, qf, a.q_scale, ntok, j4, m_run, l_run, o, pf);
        load_page_k8<D, S>(kpool + tnext * S * D, a.k_scales + tnext * S * groups, groups, kgrp, r, j4, K);
      }
      // this page's V scales -> LDS as [group][S]
#pragma unroll
      for (int y = 0; y < S * 8 / kWave; ++y) {
        const int x = y * kWave + lane;
        if (x < S * groups) vw[(x & (groups - 1)) * S + (x >> gshift)] = V.vs[y];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      page_values8<D, S>(V, ntok, j4, pf, vw, ctgrp, o);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      load_page_v8<D, S>(vpool + tnext * D * S, a.v_scales + tnext * S * groups, groups, r, j4, lane, V);
    }
  }
  wg_merge_write<D, NW>(a, b, g, split, wave, r, j4, m_run, l_run, o, mg_m, mg_l, mg_o);
}

// ---------------------------------------------------------------------------
// VALU kernel (fp32, fp8, bf16 with 16-token blocks)
// ---------------------------------------------------------------------------

// GM: an upper bound on G (8 or 16) that sizes the per-head register arrays.
template <int QK, int KVK, int D, int S, int GM>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a) {
  constexpr int LPT = kWave / S;  // lanes per token in the score phase
  constexpr int CPL = D / LPT;    // channels per lane in the score phase
  constexpr int EB = elem_bytes<KVK>();
  constexpr int VEC = Vec16<KVK>::N;
  static_assert(CPL % VEC == 0, "channel split must be whole 16-byte vectors");
  constexpr int KL = CPL / VEC;         // 16-byte K loads per lane
  constexpr int VPL = D / kWave;        // channels per lane in the value phase
  constexpr int VL = S * EB / 16;       // 16-byte loads per V channel row
  constexpr int VT = S < 32 ? S : 32;   // tokens per channel-major run of the V tile
  constexpr int TPV = 16 / EB;          // tokens per 16-byte load (divides VT)
  static_assert(VT % TPV == 0, "a V load stays inside one run");
  static_assert(VL >= 1, "a V channel row must span at least 16 bytes");

  extern __shared__ float smem[];
  const int G = a.G;
  float* qs = smem;                      // [G][D]
  float* ps = qs + G * D;                // [4][G][S]
  float* vsc = ps + 4 * G * S;           // [4][S][groups] (fp8 V scales)
  const int groups = KVK == K_FP8 ? D / a.qg : 1;
  float* mg_m = vsc + 4 * S * groups;    // [4][G]
  float* mg_l = mg_m + 4 * G;            // [4][G]
  float* mg_acc = mg_l + 4 * G;          // [3][G][D]

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // the group's query rows (G*D contiguous values): a fixed-trip loop, so
  // every load is issued before the first one is waited for
  {
    const long long q0 = ((long long)b * a.Hq + (long long)g * G) * D;
    float qv[(GM * D + 255) / 256];
#pragma unroll
    for (int x = 0; x < (GM * D + 255) / 256; ++x) {
      const int i = x * 256 + tid;
      qv[x] = 0.0f;
      if (i < G * D) {
        if constexpr (QK == K_F32)
          qv[x] = static_cast<const float*>(a.q)[q0 + i];
        else
          qv[x] = __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.q)[q0 + i] << 16);
      }
    }
#pragma unroll
    for (int x = 0; x < (GM * D + 255) / 256; ++x) {
      const int i = x * 256 + tid;
      if (i < G * D) qs[i] = qv[x] * a.q_scale;
    }
  }
  __syncthreads();
  const int len = clamp_len(a, b, tid == 0 && split == 0 && g == 0);
  const int nb = (len + S - 1) / S;

  float m_run[GM], l_run[GM], acc[GM][VPL];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m_run[h] = -__builtin_inff();
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) acc[h][e] = 0.0f;
  }

  const int32_t* srow = a.sel + ((long long)b * a.Hkv + g) * a.k;
  const int i0 = split * a.bps;
  const int i1 = min(i0 + a.bps, a.k);
  const int t = lane % S, part = lane / S;
  float* pw = ps + wave * G * S;
  float* vw = vsc + wave * S * groups;
  const char* kb = static_cast<const char*>(a.k_pool);
  const char* vb = static_cast<const char*>(a.v_pool);
  const int c0 = lane * VPL;  // value-phase channels of this lane
  // the scale groups of this lane's channels, computed once (no division in the loops)
  int vgrp[VPL], kgrp[KL];
#pragma unroll
  for (int e = 0; e < VPL; ++e) vgrp[e] = KVK == K_FP8 ? (c0 + e) / a.qg : 0;
#pragma unroll
  for (int x = 0; x < KL; ++x) kgrp[x] = KVK == K_FP8 ? (part * CPL + x * VEC) / a.qg : 0;

  for (int i = i0 + wave; i < i1; i += 4) {
    int j = 0;
    const int entry = tile_entry(a, srow, i, b, g, nb, lane, &j);
    if (entry < 0) continue;
    const long long tile = a.hot ? (long long)entry : (long long)entry * a.Hkv + g;
    const long long row0 = tile * S;  // token rows of the tile
    const int ntok = min(S, len - j * S);

    // ---- all loads of the tile ----
    uint4 kraw[KL], vraw[VPL][VL];
    float ksc[KL];  // fp8: the scale of each 16-channel chunk's group, loaded with the tile
    if (t < ntok) {
#pragma unroll
      for (int x = 0; x < KL; ++x)
        kraw[x] = *reinterpret_cast<const uint4*>(kb + ((row0 + t) * D + part * CPL + x * VEC) * EB);
      if constexpr (KVK == K_FP8) {
#pragma unroll
        for (int x = 0; x < KL; ++x) ksc[x] = a.k_scales[(row0 + t) * groups + kgrp[x]];
      }
    }
#pragma unroll
    for (int e = 0; e < VPL; ++e)
#pragma unroll
      for (int x = 0; x < VL; ++x)
        vraw[e][x] = *reinterpret_cast<const uint4*>(
            vb + (tile * S * D + ((x * TPV) / VT * D + c0 + e) * VT + (x * TPV) % VT) * EB);
    if constexpr (KVK == K_FP8) {
      // at most 8 groups per token: a fixed-trip loop, all loads in flight together
      float vsv[S * 8 / kWave];
#pragma unroll
      for (int y = 0; y < S * 8 / kWave; ++y) {
        const int x = y * kWave + lane;
        vsv[y] = x < S * groups ? a.v_scales[row0 * groups + x] : 0.0f;
      }
#pragma unroll
      for (int y = 0; y < S * 8 / kWave; ++y) {
        const int x = y * kWave + lane;
        if (x < S * groups) vw[x] = vsv[y];
      }
    }

    // ---- scores (lane = token) ----
    float dot[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) dot[h] = 0.0f;
    if (t < ntok) {
#pragma unroll
      for (int x = 0; x < KL; ++x) {
        const int c = part * CPL + x * VEC;
        float kv[VEC];
        const uint32_t ws[4] = {kraw[x].x, kraw[x].y, kraw[x].z, kraw[x].w};
        if constexpr (KVK == K_F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) kv[e] = __uint_as_float(ws[e]);
        } else if constexpr (KVK == K_BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[2 * e] = bf16_lo(ws[e]);
            kv[2 * e + 1] = bf16_hi(ws[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) fp8x4_to_f32(ws[e], kv + 4 * e);
          const float sc = ksc[x];
#pragma unroll
          for (int e = 0; e < VEC; ++e) kv[e] *= sc;
        }
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          if (h < G) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
              const float4 qv = *reinterpret_cast<const float4*>(qs + h * D + c + e);
              dot[h] += qv.x * kv[e] + qv.y * kv[e + 1] + qv.z * kv[e + 2] + qv.w * kv[e + 3];
            }
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
#pragma unroll
        for (int off = S; off < kWave; off <<= 1) dot[h] += __shfl_xor(dot[h], off);
      }
    }
    // ---- online softmax (base 2) ----
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float s = t < ntok ? dot[h] : -__builtin_inff();
        const float mt = wave_max(s);
        const float mnew = fmaxf(m_run[h], mt);
        const float alpha = exp2f(m_run[h] - mnew);
        const float p = exp2f(s - mnew);
        const float psum = wave_sum(part == 0 ? p : 0.0f);
        l_run[h] = l_run[h] * alpha + psum;
        m_run[h] = mnew;
#pragma unroll
        for (int e = 0; e < VPL; ++e) acc[h][e] *= alpha;
        if (part == 0) pw[h * S + t] = p;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- values (lane = channel), converted four tokens at a time ----
    constexpr int PER = 16 / EB;  // tokens per 16-byte load
#pragma unroll
    for (int tt = 0; tt < S; tt += 4) {
      float v[VPL][4];
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        const uint4 w4 = vraw[e][tt / PER];
        const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
        const int o4 = tt % PER;
        if constexpr (KVK == K_F32) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[e][q] = __uint_as_float(ws[q]);
        } else if constexpr (KVK == K_BF16) {
          v[e][0] = bf16_lo(ws[o4 / 2]);
          v[e][1] = bf16_hi(ws[o4 / 2]);
          v[e][2] = bf16_lo(ws[o4 / 2 + 1]);
          v[e][3] = bf16_hi(ws[o4 / 2 + 1]);
        } else {
          fp8x4_to_f32(ws[o4 / 4], v[e]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float vv = v[e][q];
          if constexpr (KVK == K_FP8) vv *= vw[(tt + q) * groups + vgrp[e]];
          v[e][q] = tt + q < ntok ? vv : 0.0f;
        }
      }
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const float4 p4 = *reinterpret_cast<const float4*>(pw + h * S + tt);
#pragma unroll
          for (int e = 0; e < VPL; ++e)
            acc[h][e] += p4.x * v[e][0] + p4.y * v[e][1] + p4.z * v[e][2] + p4.w * v[e][3];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the four wavefronts ----
  if (lane == 0) {
    for (int h = 0; h < G; ++h) {
      mg_m[wave * G + h] = m_run[h];
      mg_l[wave * G + h] = l_run[h];
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h)
      if (h < G)
#pragma unroll
        for (int e = 0; e < VPL; ++e) mg_acc[((wave - 1) * G + h) * D + c0 + e] = acc[h][e];
  }
  __syncthreads();
  if (wave == 0) {
    const bool direct = a.nsplit == 1;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h >= G) continue;
      float M = mg_m[h];
#pragma unroll
      for (int w = 1; w < 4; ++w) M = fmaxf(M, mg_m[w * G + h]);
      float sc[4];
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = mg_m[w * G + h];
        sc[w] = mw == -__builtin_inff() ? 0.0f : exp2f(mw - M);
        L += mg_l[w * G + h] * sc[w];
      }
      const float inv = direct ? (L > 0.0f ? 1.0f / L : 0.0f) : 1.0f;
      const long long hrow = (long long)b * a.Hq + (long long)g * G + h;
      const long long pi = hrow * a.nsplit + split;
      if (!direct && lane == 0) {
        a.part_m[pi] = M;
        a.part_l[pi] = L;
      }
      float* dst = direct ? a.out + hrow * D : a.part_acc + pi * D;
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        float o = acc[h][e] * sc[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) o += mg_acc[((w - 1) * G + h) * D + c0 + e] * sc[w];
        dst[c0 + e] = o * inv;
      }
    }
  }
}

// Split merge: one thread per (query head, 4 output channels), 64 threads
// per workgroup.  Each thread loads, in one round trip, the head's split
// maxima and normalisers (the same addresses for the head's threads) and its
// 4 channels of every split's partial, in batches of kMergeBatch splits, and
// merges them online in registers:
//   M = max m_i, L = sum l_i 2^(m_i - M), o = sum acc_i 2^(m_i - M) / L.
// No cross-lane traffic and no barriers.
constexpr int kMaxSplits = kComputeUnits;  // attn_num_splits never exceeds it
constexpr int kMergeThreads = 64;
constexpr int kMergeBatch = 8;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnArgs a) {
  constexpr int C4 = D / 4;  // float4 chunks per head
  // numbered like the attention's workgroups (xcd_unit), so that a unit's
  // heads tend to be merged on the XCD whose L2 took its split partials
  const long long t = (long long)xcd_order(blockIdx.x, gridDim.x) * kMergeThreads + threadIdx.x;
  const long long nrows = (long long)a.B * a.Hq;
  if (t >= nrows * C4) return;
  const long long row = t / C4;
  const int c = (int)(t % C4) * 4;
  const int ns = a.nsplit;
  const float* pm = a.part_m + row * ns;
  const float* pl = a.part_l + row * ns;
  const float* pa = a.part_acc + row * ns * D + c;
  float M = -__builtin_inff(), Ls = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch];
    float4 av[kMergeBatch];
#pragma unroll
    for (int x = 0; x < kMergeBatch; ++x) {
      const int s = s0 + x;
      mv[x] = -__builtin_inff();
      lv[x] = 0.0f;
      av[x] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (s < ns) {
        mv[x] = pm[s];
        lv[x] = pl[s];
        av[x] = *reinterpret_cast<const float4*>(pa + (long long)s * D);
      }
    }
    float Mb = M;
#pragma unroll
    for (int x = 0; x < kMergeBatch; ++x) Mb = fmaxf(Mb, mv[x]);
    if (Mb == -__builtin_inff()) continue;  // nothing valid yet
    const float sc = M == -__builtin_inff() ? 0.0f : exp2f(M - Mb);
    Ls *= sc;
    acc.x *= sc;
    acc.y *= sc;
    acc.z *= sc;
    acc.w *= sc;
#pragma unroll
    for (int x = 0; x < kMergeBatch; ++x) {
      const float wgt = mv[x] == -__builtin_inff() ? 0.0f : exp2f(mv[x] - Mb);
      Ls += lv[x] * wgt;
      acc.x += wgt * av[x].x;
      acc.y += wgt * av[x].y;
      acc.z += wgt * av[x].z;
      acc.w += wgt * av[x].w;
    }
    M = Mb;
  }
  const float inv = (M != -__builtin_inff() && Ls > 0.0f) ? 1.0f / Ls : 0.0f;
  *reinterpret_cast<float4*>(a.out + row * D + c) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

template <int QK, int KVK, int D, int GM>
void launch_valu_s(const AttnArgs& a, size_t lds, hipStream_t st) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)a.B);
  switch (a.S) {
    case 16: hipLaunchKernelGGL((attn_valu_kernel<QK, KVK, D, 16, GM>), grid, dim3(256), lds, st, a); break;
    case 32: hipLaunchKernelGGL((attn_valu_kernel<QK, KVK, D, 32, GM>), grid, dim3(256), lds, st, a); break;
    default: hipLaunchKernelGGL((attn_valu_kernel<QK, KVK, D, 64, GM>), grid, dim3(256), lds, st, a); break;
  }
}

template <int QK, int KVK, int D>
hipError_t launch_valu(const AttnArgs& a, hipStream_t st) {
  const int groups = KVK == K_FP8 ? D / a.qg : 1;
  const size_t lds = sizeof(float) * ((size_t)a.G * D + 4 * (size_t)a.G * a.S + 4 * (size_t)a.S * groups +
                                      8 * (size_t)a.G + 3 * (size_t)a.G * D);
  if (a.G <= 8)
    launch_valu_s<QK, KVK, D, 8>(a, lds, st);
  else
    launch_valu_s<QK, KVK, D, kGMax>(a, lds, st);
  return hipGetLastError();
}

template <int D, int SELF, int PG>
void launch_mfma8_g(const AttnArgs& a, const dim3& grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_mfma8_kernel<D, kAttnTile, kAttnWaves, SELF, PG>), grid, dim3(64 * kAttnWaves), 0, st, a);
}
template <int D, int SELF>
void launch_mfma8_s(const AttnArgs& a, const dim3& grid, hipStream_t st) {
  if (a.qg >= 32)
    launch_mfma8_g<D, SELF, 1>(a, grid, st);
  else
    launch_mfma8_g<D, SELF, 0>(a, grid, st);
}

template <int D>
hipError_t launch_mfma8(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)a.B);
  if (!a.W)
    launch_mfma8_s<D, 0>(a, grid, st);
  else if (a.MB <= 512)
    launch_mfma8_s<D, 2>(a, grid, st);
  else
    launch_mfma8_s<D, kSelfSelMax / 256>(a, grid, st);
  return hipGetLastError();
}

template <int D, int SELF>
void launch_mfma_s(const AttnArgs& a, const dim3& grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_mfma_kernel<D, kAttnTile, kAttnWaves, SELF>), grid, dim3(64 * kAttnWaves), 0, st, a);
}

template <int D>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)a.B);
  if (!a.W)
    launch_mfma_s<D, 0>(a, grid, st);
  else if (a.MB <= 512)
    launch_mfma_s<D, 2>(a, grid, st);
  else
    launch_mfma_s<D, kSelfSelMax / 256>(a, grid, st);
  return hipGetLastError();
}

}  // namespace

int attn_num_splits(int units, int k) {
  // As few splits as still give about one workgroup per compute unit: each
  // wavefront then streams the most pages through its pipeline, and the
  // split partials to merge are fewest (one split writes the output).
  // Measured on the 8 x 4 unit, k = 128 shape: 2/4/6/8 pages per wavefront
  // take 37.0/33.5/36.2/44.4 us; on 256 x 4, k = 32: 4 pages 221 us, 8 pages
  // (one split) 199 us.
  if (units < 1) units = 1;
  const int by_k = (k + 3) / 4;  // at least one page per wavefront
  const int want = (kComputeUnits + units - 1) / units;
  const int n = by_k < want ? by_k : want;
  return n < 1 ? 1 : n;
}

bool attn_self_select_supported(int q_kind, int kv_kind, int S, int MB, int k) {
  // the matrix-core kernels (bf16 q; bf16 or fp8 K/V; S >= 32) carry the
  // selection prologue
  return q_kind == K_BF16 && (kv_kind == K_BF16 || kv_kind == K_FP8) && S >= 32 && MB <= kSelfSelMax &&
         k <= kSelfSelMax;
}

bool attn_tok_supported(int q_kind, int kv_kind, int S, int D, int hot) {
  return q_kind == K_BF16 && kv_kind == K_BF16 && S >= 32 && (D == 64 || D == 128) && !hot;
}

hipError_t launch_attn_tok(const AttnArgs& a, const AppendArgs& t, int q_kind, int kv_kind, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.nsplit < 1 || a.nsplit > kMaxSplits || a.W || !attn_tok_supported(q_kind, kv_kind, a.S, a.D, a.hot))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)a.B);
  if (a.D == 64)
    hipLaunchKernelGGL((attn_mfma_tok_kernel<64, kAttnTile, kAttnWaves>), grid, dim3(64 * kAttnWaves), 0, st, a, t);
  else
    hipLaunchKernelGGL((attn_mfma_tok_kernel<128, kAttnTile, kAttnWaves>), grid, dim3(64 * kAttnWaves), 0, st, a, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const long long threads = (long long)a.B * a.Hq * (a.D / 4);
  const dim3 mgrid((unsigned)((threads + kMergeThreads - 1) / kMergeThreads));
  if (a.D == 64)
    hipLaunchKernelGGL(merge_kernel<64>, mgrid, dim3(kMergeThreads), 0, st, a);
  else
    hipLaunchKernelGGL(merge_kernel<128>, mgrid, dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, int q_kind, int kv_kind, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.nsplit < 1 || a.nsplit > kMaxSplits) return hipErrorInvalidValue;  // merge_kernel's bound
  if (a.W && !attn_self_select_supported(q_kind, kv_kind, a.S, a.MB, a.k)) return hipErrorInvalidValue;
  hipError_t e;
  if (q_kind == K_BF16 && kv_kind == K_BF16 && a.S >= 32)
    e = a.D == 64 ? launch_mfma<64>(a, st) : launch_mfma<128>(a, st);
  else if (q_kind == K_F32 && kv_kind == K_F32)
    e = a.D == 64 ? launch_valu<K_F32, K_F32, 64>(a, st) : launch_valu<K_F32, K_F32, 128>(a, st);
  else if (q_kind == K_BF16 && kv_kind == K_FP8 && a.S >= 32)
    e = a.D == 64 ? launch_mfma8<64>(a, st) : launch_mfma8<128>(a, st);
  else if (q_kind == K_BF16 && kv_kind == K_BF16)
    e = a.D == 64 ? launch_valu<K_BF16, K_BF16, 64>(a, st) : launch_valu<K_BF16, K_BF16, 128>(a, st);
  else
    e = a.D == 64 ? launch_valu<K_BF16, K_FP8, 64>(a, st) : launch_valu<K_BF16, K_FP8, 128>(a, st);
  if (e != hipSuccess || a.nsplit == 1) return e;
  const long long threads = (long long)a.B * a.Hq * (a.D / 4);
  const dim3 grid((unsigned)((threads + kMergeThreads - 1) / kMergeThreads));
  if (a.D == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeThreads), 0, st, a);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvs
