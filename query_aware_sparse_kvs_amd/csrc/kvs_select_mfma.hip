// kvs_select_mfma.hip -- block scores on the matrix cores and the exact
// top-k (page "KV 稀疏化", §5 "Quest": coarse-filter the blocks with the
// query and the summaries, keep the top-k; the sink and the newest block are
// always kept).  bf16 query; bf16 summaries, or fp32 summaries (of fp8 K,
// "分块稀疏注意力与KV Cache量化…" §1.3) split into two bf16 parts;
// identical selections to the all-exact path in kvs_select.hip, at a
// fraction of its arithmetic.
//
// scores32_kernel -- fp32 scores of every block on the matrix cores.  With
// q+ = max(q, 0) and q- = min(q, 0) the box bound is
//   U[j,h] = sum_c q+_hc * max_jc + q-_hc * min_jc,
// the product of a [16 blocks x 2D] summary tile and the [2D x 16 heads]
// query tile (heads padded to 16): 2D/32 v_mfma_f32_16x16x32_bf16 per 16
// blocks.  bf16 x bf16 products are exact; the sums are fp32.  The same
// product over absolute values gives A[j,h] = sum_c |q_hc| |x_jc|.  Stored per
// block: W32 = max_h U32 and A = max_h A[j,h].  Four wavefronts per
// workgroup, 16 blocks each: the read of the summaries is spread over the
// whole chip (HBM-bound).  fp32 summaries: each element x is split into
// x_hi = bf16(x) and x_lo = bf16(x - x_hi) (x - x_hi is exact in fp32), so
// |x - x_hi - x_lo| <= 2^-17 |x| for normal parts; the score product runs on
// both parts (2 x 2D terms per sum) and A on |x_hi|.
//
// refine_kernel -- one 512-thread workgroup per (sequence, KV head).
// |W32 - W| <= eps = 2^-13 * max A (+ a floor for underflow) bounds the
// rounding of the 2D-term fp32 sums (an eight-fold margin over the worst
// case).  fp32 summaries: 4D-term sums (<= 2^-15 relative), the split's
// residual (<= 2^-17) and |x| <= (1 + 2^-8)|x_hi| give eps = 2^-11 * max A
// (again about eight-fold).  Both kinds add max|q| * 2^-116 for summary
// values or parts below the normal range (flushed or rounded by the matrix
// unit: at most 2 x 2D terms of |q| * 2^-126) and the 2^-110 floor.  A
// score or magnitude that is not finite (fp32 overflow), or a query value
// below the normal range (whose products could be lost whole), makes every
// candidate of the unit uncertain, so the exact chain decides.  A radix select over the candidates' (blocks 1..nb-R-1, R newest
// blocks always kept) W32 gives the
// M-th and (M+1)-th largest values vM, vM1 (M = k-1-R): a block with
// W32 > vM1 + 2*eps is in the exact top M, one with W32 < vM - 2*eps is not.
// Only the blocks in between (a handful) get their bound recomputed exactly
// -- fp64, ascending channels, the sum of the plain definition -- one thread
// per (block, head), and are ranked by (W desc, id asc) for the places left.
// The selection therefore equals the one the exact scores give.
#include <type_traits>

#include "kvs_append.h"
#include "kvs_summarize.h"

namespace kvs {
namespace {

constexpr int kFT = 512;           // threads per workgroup
constexpr int kFW = kFT / kWave;   // wavefronts
constexpr int kFMaxBlocks = 2048;  // largest max_blocks this kernel takes
constexpr int kFPT = kFMaxBlocks / kFT;  // block ids per thread

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// order-preserving map of a float (no NaN) to uint32; -0 and +0 coincide
__device__ __forceinline__ unsigned order_u32(float w) {
  const unsigned u = __float_as_uint(w + 0.0f);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_u32(unsigned k) {
  return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k);
}

// Eight fp32 values -> x_hi = bf16(x) and x_lo = bf16(x - x_hi), both
// round-to-nearest-even (x - x_hi is exact in fp32).
__device__ __forceinline__ void split_hi_lo(u32x4 w0, u32x4 w1, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = __uint_as_float(e < 4 ? w0[e] : w1[e - 4]);
    const __bf16 h = static_cast<__bf16>(x);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(x - static_cast<float>(h));
  }
}

// q+ / q- (and their absolute values) of 8 bf16 query values, bitwise
__device__ __forceinline__ void split_sign(u32x4 q, u32x4& pos, u32x4& neg, u32x4& negabs) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const unsigned w = q[e];
    const unsigned m = ((w & 0x8000u) ? 0x0000FFFFu : 0u) | ((w & 0x80000000u) ? 0xFFFF0000u : 0u);
    pos[e] = w & ~m;
    neg[e] = w & m;
    negabs[e] = (w & m) & 0x7FFF7FFFu;
  }
}

// Block-wide exclusive prefix sum over kFT threads; `tmp` holds kFW ints of
// LDS used by this call only (no barrier is needed after it).
__device__ __forceinline__ int scan_512(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kFW; ++w) {
    const int t = tmp[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + incl - v;
}

// ---------------------------------------------------------------------------
// scores32_kernel: grid (MB/64 chunks, Hkv, B), 256 threads
// ---------------------------------------------------------------------------
// SK: summary kind, K_BF16 or K_F32 (fp32 summaries come with fp8 K for a
// bf16 query)
template <int D, int SK>
__global__ __launch_bounds__(256, SK == K_BF16 ? 4 : 2) void scores32_kernel(SelMfmaArgs a) {
  constexpr int HC = D / 32;  // 32-channel chunks per summary half
  constexpr int KC = 2 * HC;  // chunks of the [max | min] row
  constexpr int KVK = SK == K_BF16 ? K_BF16 : K_FP8;
  const int g = blockIdx.y, b = blockIdx.z;
  if (a.append && blockIdx.x == gridDim.x - 1) {  // uniform: this workgroup refreshes a summary
    __shared__ float red[kSummRed<D>];
    if (a.append == 2)  // the decode token: written, folded into its block's summary
      append_token_unit<KVK, D, 256>(a.tok, b, g);
    else
      rebuild_newest_summary<KVK, D>(a.app, b, g, red);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, j4 = lane >> 4;
  const int G = a.G, MB = a.MB;
  const int jt = (blockIdx.x * 4 + wave) * 16;  // this wavefront's 16 blocks
  if (jt >= MB) return;  // uniform over the wavefront; no barrier below
  constexpr int EB = SK == K_BF16 ? 2 : 4;  // summary element bytes
  constexpr int NV = EB / 2;                // 16-byte vectors per 8 elements
  const char* summ = static_cast<const char*>(a.summ) + ((long long)b * a.Hkv + g) * MB * 2 * D * EB;
  const uint16_t* qrow0 = static_cast<const uint16_t*>(a.q) + ((long long)b * a.Hq + (long long)g * G) * D;
  // A operand (summary rows, max half first) before anything else.  Every
  // load is unconditional, so they all go out in one batch: a row past MB
  // reads row MB-1 and a head past G reads head G-1 instead; the products
  // of those rows and columns are never stored.
  u32x4 ar[KC][NV];
  const int j = min(jt + r, MB - 1);
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const int off = kc < HC ? D + kc * 32 : (kc - HC) * 32;
#pragma unroll
    for (int v = 0; v < NV; ++v)
      ar[kc][v] = *reinterpret_cast<const u32x4*>(summ + ((long long)j * 2 * D + off + 8 * j4) * EB + 16 * v);
  }
  u32x4 qv[HC];
  const int rq = min(r, G - 1);
#pragma unroll
  for (int cs = 0; cs < HC; ++cs) qv[cs] = *reinterpret_cast<const u32x4*>(qrow0 + (long long)rq * D + cs * 32 + 8 * j4);
  __builtin_amdgcn_sched_barrier(0);  // every load out before any product
  u32x4 qs[KC];  // B operand: [q+ | q-] of head r
#pragma unroll
  for (int cs = 0; cs < HC; ++cs) {
    u32x4 neg, negabs;
    split_sign(qv[cs], qs[cs], neg, negabs);
    qs[HC + cs] = neg;
  }
  f32x4_t u = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, ab = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    if constexpr (SK == K_BF16) {
      u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ar[kc][0]), as_bf(qs[kc]), u, 0, 0, 0);
      ab = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ar[kc][0] & 0x7FFF7FFFu), as_bf(qs[kc] & 0x7FFF7FFFu), ab,
                                                   0, 0, 0);
    } else {
      bf16x8_t hi, lo;
      split_hi_lo(ar[kc][0], ar[kc][NV - 1], hi, lo);
      u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, as_bf(qs[kc]), u, 0, 0, 0);
      u = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, as_bf(qs[kc]), u, 0, 0, 0);
      ab = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(__builtin_bit_cast(u32x4, hi) & 0x7FFF7FFFu),
                                                   as_bf(qs[kc] & 0x7FFF7FFFu), ab, 0, 0, 0);
    }
  }
  // lane (r, j4) holds blocks jt + 4*j4 + e of head r: max over the heads
  float* w32 = a.w32 + ((long long)b * a.Hkv + g) * MB;
  float* amag = a.amag + ((long long)b * a.Hkv + g) * MB;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = r < G ? u[e] : -__builtin_inff();
    float m = r < G ? ab[e] : 0.0f;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      v = fmaxf(v, __shfl_xor(v, off));
      m = fmaxf(m, __shfl_xor(m, off));
    }
    const int jj = jt + 4 * j4 + e;
    if (r == 0 && jj < MB) {
      w32[jj] = v;
      amag[jj] = m;
    }
  }
}

// ---------------------------------------------------------------------------
// refine_kernel: grid (Hkv, B), 512 threads
// ---------------------------------------------------------------------------
template <int D, int SK>
__global__ __launch_bounds__(kFT) void refine_kernel(SelMfmaArgs a) {
  constexpr int UB = kFT / 16;  // uncertain blocks per exact round (16 threads each)
  using SE = std::conditional_t<SK == K_BF16, uint16_t, float>;  // summary element
  __shared__ unsigned char flag[kFMaxBlocks];  // 3: uncertain and chosen
  __shared__ int ulist[kFMaxBlocks];
  __shared__ double uw[kFMaxBlocks];
  __shared__ float qf[16][D + 1];
  __shared__ __attribute__((aligned(16))) SE rowbuf[UB][2 * D];
  __shared__ unsigned hist[2][256];
  __shared__ float red_f[kFW], red_q[kFW];
  __shared__ unsigned red_u[2][kFW];
  __shared__ unsigned red_b[kFW];
  __shared__ int scan_a[kFW], scan_b[kFW], scan_c[kFW];
  __shared__ unsigned sh_T[2];
  __shared__ int sh_rem[2];

  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.G, k = a.k, MB = a.MB;
  const float* w32g = a.w32 + ((long long)b * a.Hkv + g) * MB;
  const float* amag = a.amag + ((long long)b * a.Hkv + g) * MB;
  const SE* summ = static_cast<const SE*>(a.summ) + ((long long)b * a.Hkv + g) * MB * 2 * D;
  const uint16_t* qrow0 = static_cast<const uint16_t*>(a.q) + ((long long)b * a.Hq + (long long)g * G) * D;

  // ---- every load first: this thread's scores and magnitudes, the length, q ----
  const int j0 = tid * kFPT;  // this thread's contiguous block ids
  float wv[kFPT], am[kFPT];
#pragma unroll
  for (int i = 0; i < kFPT; ++i) {
    const bool in = j0 + i < MB;
    wv[i] = in ? w32g[j0 + i] : 0.0f;
    am[i] = in ? amag[j0 + i] : 0.0f;
  }
  int len = a.seq_lens[b];
  float qmax = 0.0f;  // the largest |q| of the group (a floor of eps)
  int qsub = 0;       // a query value below the normal range (its products may be lost whole)
  for (int i = tid; i < G * D; i += kFT) {
    const float qv = __uint_as_float((uint32_t)qrow0[i] << 16);
    qf[i / D][i % D] = qv;
    qmax = fmaxf(qmax, fabsf(qv));
    if (qv != 0.0f && fabsf(qv) < 0x1p-126f) qsub = 1;
  }
  if (tid < 256) hist[0][tid] = 0u;
  const int cap = MB * a.S;
  if (len < 0 || len > cap) {
    if (tid == 0 && g == 0) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  const int nb = (len + a.S - 1) / a.S;
  int32_t* out = a.sel + ((long long)b * a.Hkv + g) * k;
  if (nb <= k) {  // every block, then padding
    for (int i = tid; i < k; i += kFT) out[i] = i < nb ? i : -1;
    return;
  }
  const int RW = a.recent;
  const int M = k - 1 - RW;  // places besides the sink and the RW newest blocks
  if (M == 0) {
    for (int i = tid; i < k; i += kFT) out[i] = i == 0 ? 0 : nb - RW + (i - 1);
    return;
  }

  // ---- candidates, their order keys; eps and the key range in one reduction ----
  bool cand[kFPT];
  unsigned key[kFPT];
  unsigned kmin = 0xFFFFFFFFu, kmax = 0u;
  float amax = 0.0f;
  int bad = qsub;  // a score or magnitude that is not finite, or a subnormal query value
#pragma unroll
  for (int i = 0; i < kFPT; ++i) {
    const int j = j0 + i;
    cand[i] = j >= 1 && j < nb - RW;
    if (cand[i] && !(__builtin_isfinite(wv[i]) && __builtin_isfinite(am[i]))) bad = 1;
    key[i] = cand[i] && __builtin_isfinite(wv[i]) ? order_u32(wv[i]) : 0u;
    if (cand[i]) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
      amax = fmaxf(amax, am[i]);
    }
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    kmin = min(kmin, (unsigned)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (unsigned)__shfl_xor((int)kmax, off));
    amax = fmaxf(amax, __shfl_xor(amax, off));
    qmax = fmaxf(qmax, __shfl_xor(qmax, off));
    bad |= __shfl_xor(bad, off);
  }
  if (lane == 0) {
    red_u[0][wave] = kmin;
    red_u[1][wave] = kmax;
    red_f[wave] = amax;
    red_q[wave] = qmax;
    red_b[wave] = (unsigned)bad;
  }
  __syncthreads();
  unsigned kmn = red_u[0][0], kmx = red_u[1][0];
  amax = red_f[0];
  qmax = red_q[0];
  bad = (int)red_b[0];
#pragma unroll
  for (int w = 1; w < kFW; ++w) {
    kmn = min(kmn, red_u[0][w]);
    kmx = max(kmx, red_u[1][w]);
    amax = fmaxf(amax, red_f[w]);
    qmax = fmaxf(qmax, red_q[w]);
    bad |= (int)red_b[w];
  }
  __syncthreads();  // red_b is reused below
  // (the floors cover products below 2^-126 flushed, and summary parts below
  // the normal range lost, over all terms; the fp32-summary terms are derived
  // in the header comment)
  const float eps = (SK == K_BF16 ? amax * 0x1p-13f : amax * 0x1p-11f) + qmax * 0x1p-116f + 0x1p-110f;

  // ---- radix select of the M-th largest key (8-bit digits, from the first
  // differing byte; two histograms alternate so one barrier separates the
  // count from the search and one the search from the next count) ----
  unsigned T = kmn;
  int rem = M;
  if (kmn != kmx) {
    const int top_bit = 31 - __clz(kmn ^ kmx);
    unsigned mask = top_bit / 8 >= 3 ? 0u : (0xFFFFFFFFu << (8 * (top_bit / 8 + 1)));
    unsigned prefix = kmn & mask;
    int hb = 0;
    for (int pass = top_bit / 8; pass >= 0; --pass, hb ^= 1) {
      const int shift = pass * 8;
#pragma unroll
      for (int i = 0; i < kFPT; ++i)
        if (cand[i] && (key[i] & mask) == prefix) atomicAdd(&hist[hb][(key[i] >> shift) & 255u], 1u);
      if (tid < 256) hist[hb ^ 1][tid] = 0u;  // the next pass's histogram
      __syncthreads();
      if (tid < 64) {
        unsigned c4[4], s = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c4[e] = hist[hb][255 - 4 * tid - e];
          s += c4[e];
        }
        unsigned incl = s;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const unsigned o = __shfl_up(incl, off);
          if (tid >= off) incl += o;
        }
        unsigned above = incl - s;
        if ((int)above < rem && rem <= (int)incl) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((int)(above + c4[e]) >= rem) {
              sh_T[hb] = prefix | ((unsigned)(255 - 4 * tid - e) << shift);
              sh_rem[hb] = rem - (int)above;
              break;
            }
            above += c4[e];
          }
        }
      }
      __syncthreads();
      prefix = sh_T[hb];
      rem = sh_rem[hb];
      mask |= 0xFFu << shift;
    }
    T = prefix;
  }
  const int rem_eq = rem;  // how many keys equal to T the top M takes

  // ---- keys equal to T, and the largest key below it (one reduction) ----
  int n_eq_local = 0;
  unsigned below = 0u;  // order keys are > 0 for every finite score, so 0 = none
#pragma unroll
  for (int i = 0; i < kFPT; ++i) {
    if (!cand[i]) continue;
    if (key[i] == T) ++n_eq_local;
    if (key[i] < T) below = max(below, key[i]);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    n_eq_local += __shfl_xor(n_eq_local, off);
    below = max(below, (unsigned)__shfl_xor((int)below, off));
  }
  if (lane == 0) {
    scan_c[wave] = n_eq_local;
    red_b[wave] = below;
  }
  __syncthreads();
  int n_eq = 0;
  below = 0u;
#pragma unroll
  for (int w = 0; w < kFW; ++w) {
    n_eq += scan_c[w];
    below = max(below, red_b[w]);
  }
  const float vM = from_order_u32(T);
  const float vM1 = rem_eq < n_eq ? vM : (below ? from_order_u32(below) : -__builtin_inff());
  const double lo_cut = (double)vM - 2.0 * (double)eps;
  const double hi_cut = (double)vM1 + 2.0 * (double)eps;

  // ---- certain in (1), uncertain (2); positions of the uncertain ones ----
  int n_in_local = 0, n_u_local = 0;
  unsigned char cls[kFPT];
#pragma unroll
  for (int i = 0; i < kFPT; ++i) {
    cls[i] = 0;
    if (!cand[i]) continue;
    const double w = (double)wv[i];
    if (bad) {  // no usable estimate: every candidate is ranked exactly
      cls[i] = 2;
      ++n_u_local;
    } else if (w > hi_cut) {
      cls[i] = 1;
      ++n_in_local;
    } else if (w >= lo_cut) {
      cls[i] = 2;
      ++n_u_local;
    }
  }
  int packed_tot;
  const int packed = scan_512(n_in_local | (n_u_local << 16), scan_a, &packed_tot);
  const int n_in = packed_tot & 0xFFFF, n_u = packed_tot >> 16;
  int upos = packed >> 16;
#pragma unroll
  for (int i = 0; i < kFPT; ++i) {
    const int j = j0 + i;
    if (j < MB) flag[j] = cls[i];
    if (cls[i] == 2) ulist[upos++] = j;
  }
  const int R = M - n_in;  // places left for uncertain blocks, 0 <= R <= n_u
  __syncthreads();

  // ---- exact scores of the uncertain blocks, only when they must be ranked ----
  if (R > 0 && R < n_u) {
    for (int u0 = 0; u0 < n_u; u0 += UB) {
      const int nu = min(UB, n_u - u0);
      constexpr int EPV = 16 / sizeof(SE);  // elements per 16-byte vector
      constexpr int V16 = 2 * D / EPV;       // 16-byte vectors per summary row
      for (int x = tid; x < nu * V16; x += kFT) {
        const int uu = x / V16, c8 = (x % V16) * EPV;
        *reinterpret_cast<u32x4*>(&rowbuf[uu][c8]) =
            *reinterpret_cast<const u32x4*>(summ + (long long)ulist[u0 + uu] * 2 * D + c8);
      }
      __syncthreads();
      const int uu = tid / 16, h = tid % 16;
      double acc = -__builtin_inf();
      if (uu < nu && h < G) {
        acc = 0.0;
        for (int c0 = 0; c0 < D; c0 += 8) {  // 16-byte reads, the chain still in ascending c
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float qc = qf[h][c0 + e];
            float mn, mx;
            if constexpr (SK == K_BF16) {
              mn = bf16_lo(rowbuf[uu][c0 + e]);
              mx = bf16_lo(rowbuf[uu][D + c0 + e]);
            } else {
              mn = rowbuf[uu][c0 + e];
              mx = rowbuf[uu][D + c0 + e];
            }
            acc = __builtin_fma((double)qc, (double)(qc >= 0.0f ? mx : mn), acc);
          }
        }
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const double o = __shfl_xor(acc, off);
        acc = o > acc ? o : acc;
      }
      if (h == 0 && uu < nu) uw[u0 + uu] = acc;
      __syncthreads();
    }
    // rank each uncertain block among the uncertain ones: (W desc, id asc)
    for (int u = tid; u < n_u; u += kFT) {
      const double wu = uw[u];
      const int ju = ulist[u];
      int rank = 0;
      for (int v = 0; v < n_u; ++v) {
        const double wx = uw[v];
        rank += (wx > wu || (wx == wu && ulist[v] < ju)) ? 1 : 0;
      }
      if (rank < R) flag[ju] = 3;
    }
    __syncthreads();
  }

  // ---- the selection in ascending order ----
  int n_sel = 0;
  unsigned chosen = 0u;
#pragma unroll
  for (int i = 0; i < kFPT; ++i) {
    const int j = j0 + i;
    if (j >= nb) continue;
    bool take;
    if (j == 0 || j >= nb - RW)
      take = true;
    else if (cls[i] == 1)
      take = true;
    else if (cls[i] == 2)
      take = R == n_u || (R > 0 && flag[j] == 3);
    else
      take = false;
    if (take) {
      chosen |= 1u << i;
      ++n_sel;
    }
  }
  int tot;
  int pos = scan_512(n_sel, scan_b, &tot);
#pragma unroll
  for (int i = 0; i < kFPT; ++i)
    if ((chosen & (1u << i)) && pos < k) out[pos++] = j0 + i;
  for (int i = tot + tid; i < k; i += kFT) out[i] = -1;
}

}  // namespace

bool select_mfma_supported(int q_kind, int summ_kind, int D, int MB, int G) {
  return q_kind == K_BF16 && (summ_kind == K_BF16 || summ_kind == K_F32) && (D == 64 || D == 128) &&
         MB <= kFMaxBlocks && G <= 16;
}

namespace {
template <int D, int SK>
void launch_select_mfma_k(const SelMfmaArgs& a, const dim3& g1, const dim3& g2, hipStream_t s) {
  hipLaunchKernelGGL((scores32_kernel<D, SK>), g1, dim3(256), 0, s, a);
  hipLaunchKernelGGL((refine_kernel<D, SK>), g2, dim3(kFT), 0, s, a);
}
}  // namespace

hipError_t launch_select_mfma(const SelMfmaArgs& a, int summ_kind, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const dim3 g1((unsigned)((a.MB + 63) / 64 + (a.append ? 1 : 0)), (unsigned)a.Hkv, (unsigned)a.B);
  const dim3 g2((unsigned)a.Hkv, (unsigned)a.B);
  if (summ_kind == K_F32) {
    if (a.D == 64)
      launch_select_mfma_k<64, K_F32>(a, g1, g2, s);
    else
      launch_select_mfma_k<128, K_F32>(a, g1, g2, s);
  } else {
    if (a.D == 64)
      launch_select_mfma_k<64, K_BF16>(a, g1, g2, s);
    else
      launch_select_mfma_k<128, K_BF16>(a, g1, g2, s);
  }
  return hipGetLastError();
}

}  // namespace kvs
