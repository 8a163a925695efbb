// kvs_select.hip -- query-aware block scores and top-k selection (page
// "KV 稀疏化", §5 "Quest": coarse-filter the blocks with the query and the
// summaries, keep the top-k; the sink block and the newest block are always
// kept, same page §2 and "SparDA：把KV選擇提前一層…" §4.2).
//
// bounds_kernel: a workgroup of 4 wavefronts (8 for bf16 summaries and
// groups of 8 or more query heads, one per head) stages 64 consecutive blocks' summaries in LDS
// with coalesced 16-byte loads; lane = block, wavefront w takes query heads
// w, w+NW, ...  The block score is
// U = sum_c max(q_c*mn_c, q_c*mx_c); since mx_c >= mn_c the larger product is
// q_c*mx_c when q_c >= 0 and q_c*mn_c otherwise.  That choice depends only
// on the head, so it is uniform over a wavefront: a per-head bit mask picks
// mn or mx for a whole 32-bit word of summaries with one bit-field insert,
// and the head's query sits in LDS as fp64 (broadcast reads).  Every product
// of a bf16/fp32 query with a bf16/fp32 summary is exact in fp64 and the sum
// runs in ascending c, so the result is bit-identical to the plain ordered
// fp64 sum.  The group max over heads goes through LDS.  Roofline: HBM read
// of the summaries (2*D*elem bytes per block and KV head); the fp64 chain
// costs about four vector instructions per (block, head, channel).
//
// topk_kernel: one 256-thread workgroup per (sequence, KV head).  Scores are
// mapped to order-preserving 64-bit keys.  A most-significant-digit radix
// select (8-bit digits, LDS histogram) over the high 32 bits, starting at
// the first bit where the candidates' keys differ, finds the bucket of the
// (k-1-R)-th largest key among blocks 1..nb-R-1 (R = the recent window, the
// newest blocks that are always kept; "SparDA…" §4.2 keeps the last 512 or
// 1024 tokens); only when that bucket holds
// more keys than are needed does a second select run on the low 32 bits of
// the tied keys.  Ties on the full key go to the lowest block ids, the
// (W desc, id asc) order.  A block-wide prefix sum writes the chosen ids in
// ascending order.  Latency-bound.
//
// With score smoothing on, the bounds kernel ranks blocks by the smoothed
// score alpha*W + (1-alpha)*history ("SparDA…" §6.1) instead of W itself.
#include "kvs_append.h"
#include "kvs_summarize.h"

namespace kvs {
namespace {

constexpr int kBoundBlocks = 64;  // blocks per bounds workgroup (lane = block)

// wavefronts per bounds workgroup: one per query head of the group, 4 to 8
// (4 with fp32 summaries, whose chunk fills half the LDS)
template <int G, int SK>
constexpr int bound_waves() {
  return G >= 8 && SK == K_BF16 ? 8 : 4;
}

// Score smoothing across decode steps ("SparDA…" §6.1): the score a block is
// ranked by is alpha * (this step's W) + (1 - alpha) * (its smoothed score of
// the previous step), or W itself when the state holds NaN (no history).
// The state keeps the result.  Each product and the sum are rounded to fp64
// separately (no fused multiply-add), as the plain definition reads.
__device__ __forceinline__ double smooth_score(double w, double* state, double alpha, double beta) {
#pragma clang fp contract(off)
  const double h = *state;
  double r = w;
  if (!__builtin_isnan(h)) {
    const double x = alpha * w;
    const double y = beta * h;
    r = x + y;
  }
  *state = r;
  return r;
}

template <int QK, int SK, int D, int G>
__global__ __launch_bounds__((64 * bound_waves<G, SK>()), (16 / bound_waves<G, SK>())) void bounds_kernel(BoundArgs a) {
  constexpr int NWB = bound_waves<G, SK>();
  constexpr int NT = 64 * NWB;
  constexpr int NB = kBoundBlocks;
  constexpr int EB = elem_bytes<SK>();
  constexpr int ROWB = 2 * D * EB;           // bytes of one block's summary
  constexpr int ROWP = ROWB + 16;            // padded LDS row (bank spread)
  constexpr int NV = NB * ROWB / 16;         // 16-byte vectors of the chunk
  constexpr int NPT = NV / NT;
  static_assert(NV % NT == 0, "whole vectors per thread");
  constexpr int VEC = 16 / EB;               // summary elements per 16 bytes
  constexpr int WPR = D * EB / 4;            // 32-bit words per half row
  __shared__ __attribute__((aligned(16))) char sm[NB * ROWP];
  __shared__ __attribute__((aligned(16))) double qd[G][D];
  __shared__ __attribute__((aligned(16))) uint32_t qm[G][WPR];
  const int b = blockIdx.z, g = blockIdx.y;
  if (a.append == 1 && blockIdx.x == gridDim.x - 1) {  // uniform: this workgroup rebuilds a summary
    static_assert(sizeof(sm) >= kSummRed<D, NT> * sizeof(float), "summary reduction fits the chunk buffer");
    float* red = reinterpret_cast<float*>(sm);
    if constexpr (SK == K_BF16) {
      rebuild_newest_summary<K_BF16, D, NT>(a.app, b, g, red);
    } else if (a.app_kv == K_FP8) {
      rebuild_newest_summary<K_FP8, D, NT>(a.app, b, g, red);
    } else {
      rebuild_newest_summary<K_F32, D, NT>(a.app, b, g, red);
    }
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j0 = blockIdx.x * NB;
  const int nmem = min(NB, a.MB - j0);  // blocks of this chunk inside the array

  // stage the chunk's summaries: every load issued before any use, and not
  // waiting for seq_lens (blocks past nb are read but never used)
  const char* src = static_cast<const char*>(a.summ) + ((((long long)b * a.Hkv + g) * a.MB + j0) * 2 * D) * EB;
  u32x4 raw[NPT];
#pragma unroll
  for (int x = 0; x < NPT; ++x) {
    const int v = x * NT + tid;
    raw[x] = u32x4{0u, 0u, 0u, 0u};
    if (v / (ROWB / 16) < nmem) raw[x] = *reinterpret_cast<const u32x4*>(src + (long long)v * 16);
  }
  // the query as fp64, and per head the words' choice of max (mask bits set) or min
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, c = i % D;
    const long long qi = ((long long)b * a.Hq + (long long)g * G + h) * D + c;
    float v;
    if constexpr (QK == K_F32)
      v = static_cast<const float*>(a.q)[qi];
    else
      v = __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.q)[qi] << 16);
    qd[h][c] = (double)v;
  }
  // the decode token is appended by the unit's first workgroup while its
  // chunk loads are in flight (a workgroup of its own would leave some
  // compute units with two scoring workgroups)
  if (a.append == 2 && blockIdx.x == 0) {
    if constexpr (SK == K_BF16)
      append_token_unit<K_BF16, D, NT>(a.tok, b, g);
    else if (a.app_kv == K_FP8)
      append_token_unit<K_FP8, D, NT>(a.tok, b, g);
    else
      append_token_unit<K_F32, D, NT>(a.tok, b, g);
  }
  int len = a.seq_lens[b];
  const int cap = a.MB * a.S;
  if (len < 0 || len > cap) {
    if (tid == 0 && blockIdx.x == 0 && g == 0) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  const int nb = (len + a.S - 1) / a.S;
#pragma unroll
  for (int x = 0; x < NPT; ++x) {
    const int v = x * NT + tid;
    if (v / (ROWB / 16) < nmem) {
      const int blk = v / (ROWB / 16), off = (v % (ROWB / 16)) * 16;
      *reinterpret_cast<u32x4*>(sm + blk * ROWP + off) = raw[x];
    }
  }
  __syncthreads();
  for (int i = tid; i < G * WPR; i += NT) {
    const int h = i / WPR, w = i % WPR;
    uint32_t m;
    if constexpr (EB == 2)
      m = (qd[h][2 * w] >= 0.0 ? 0x0000FFFFu : 0u) | (qd[h][2 * w + 1] >= 0.0 ? 0xFFFF0000u : 0u);
    else
      m = qd[h][w] >= 0.0 ? 0xFFFFFFFFu : 0u;
    qm[h][w] = m;
  }
  __syncthreads();

  constexpr int HPW = (G + NWB - 1) / NWB;  // heads per wavefront
  const bool valid = j0 + lane < nb;
  double acc[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) acc[i] = 0.0;
  const char* pmn = sm + lane * ROWP;
  const char* pmx = pmn + D * EB;
  if (wave < G) {
#pragma unroll 1
    for (int c0 = 0; c0 < D; c0 += VEC) {
      const u32x4 vmn = *reinterpret_cast<const u32x4*>(pmn + c0 * EB);
      const u32x4 vmx = *reinterpret_cast<const u32x4*>(pmx + c0 * EB);
#pragma unroll
      for (int i = 0; i < HPW; ++i) {
        const int h = wave + NWB * i;
        if (h >= G) break;
        const u32x4 m = *reinterpret_cast<const u32x4*>(&qm[h][c0 * EB / 4]);
        const u32x4 x = (vmx & m) | (vmn & ~m);
        float xf[VEC];
        if constexpr (EB == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xf[2 * e] = bf16_lo(x[e]);
            xf[2 * e + 1] = bf16_hi(x[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) xf[e] = __uint_as_float(x[e]);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[i] = __builtin_fma(qd[h][c0 + e], (double)xf[e], acc[i]);
      }
    }
  }
  __syncthreads();  // the staged rows are no longer needed: reuse them for the group max
  double* ured = reinterpret_cast<double*>(sm);  // [G][NB]
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wave + NWB * i;
    if (h < G) ured[h * NB + lane] = acc[i];
  }
  __syncthreads();
  if (wave == 0 && lane < nmem) {
    double w = -__builtin_inf();
    if (valid) {
      w = ured[lane];
#pragma unroll
      for (int h = 1; h < G; ++h) {
        const double o = ured[h * NB + lane];
        w = o > w ? o : w;
      }
    }
    const long long wi = ((long long)b * a.Hkv + g) * a.MB + j0 + lane;
    if (a.bounds_out) a.bounds_out[wi] = w;
    if (a.ema && valid) w = smooth_score(w, a.ema_state + wi, a.ema_alpha, a.ema_beta);
    a.W[wi] = w;
  }
}

// order-preserving map of a double (no NaN) to uint64; -0 and +0 coincide
__device__ __forceinline__ unsigned long long order_key(double w) {
  const double z = w + 0.0;  // -0 -> +0
  const unsigned long long u = (unsigned long long)__double_as_longlong(z);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Radix select over the active 32-bit keys of a 256-thread workgroup: finds
// the value T of the rem-th largest active key (rem is 1-based) and how many
// keys equal to T are needed (*rem_eq).  Keys share the bits above byte
// `start_byte` (given in `prefix`), so only bytes start_byte..0 are scanned.
template <int PT>
__device__ __forceinline__ void radix_select_u32(const unsigned (&key)[PT], const bool (&act)[PT], int rem,
                                                 int start_byte, unsigned prefix, unsigned* hist,
                                                 unsigned* sh_T, int* sh_rem, unsigned* T, int* rem_eq) {
  const int tid = threadIdx.x;
  unsigned mask = start_byte >= 3 ? 0u : (0xFFFFFFFFu << (8 * (start_byte + 1)));
  prefix &= mask;
  for (int pass = start_byte; pass >= 0; --pass) {
    const int shift = pass * 8;
    hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PT; ++i)
      if (act[i] && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (highest digits first)
      unsigned c4[4], s = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = hist[255 - 4 * tid - e];
        s += c4[e];
      }
      unsigned incl = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned o = __shfl_up(incl, off);
        if (tid >= off) incl += o;
      }
      unsigned above = incl - s;  // keys in higher digits
      if ((int)above < rem && rem <= (int)incl) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((int)(above + c4[e]) >= rem) {
            *sh_T = prefix | ((unsigned)(255 - 4 * tid - e) << shift);
            *sh_rem = rem - (int)above;
            break;
          }
          above += c4[e];
        }
      }
    }
    __syncthreads();
    prefix = *sh_T;
    rem = *sh_rem;
    mask |= 0xFFu << shift;
  }
  *T = prefix;
  *rem_eq = rem;
}

// block-wide min and max of v over 256 threads (tmp: 8 words of LDS)
__device__ __forceinline__ void block_min_max_256(unsigned v_min, unsigned v_max, unsigned* tmp, unsigned* mn,
                                                  unsigned* mx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    v_min = min(v_min, (unsigned)__shfl_xor((int)v_min, off));
    v_max = max(v_max, (unsigned)__shfl_xor((int)v_max, off));
  }
  if (lane == 0) {
    tmp[wave] = v_min;
    tmp[4 + wave] = v_max;
  }
  __syncthreads();
  *mn = min(min(tmp[0], tmp[1]), min(tmp[2], tmp[3]));
  *mx = max(max(tmp[4], tmp[5]), max(tmp[6], tmp[7]));
}

template <int PT>  // candidates per thread (contiguous block ids)
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ unsigned hist[256];
  __shared__ unsigned mm_tmp[8];
  __shared__ int scan_tmp[4];
  __shared__ unsigned sh_T;
  __shared__ int sh_rem;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int k = a.k;
  int len = a.seq_lens[b];
  const int cap = a.MB * a.S;
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int nb = (len + a.S - 1) / a.S;
  int32_t* out = a.sel + ((long long)b * a.Hkv + g) * k;

  // scores of every id below MB are loaded before nb is known (ids past nb
  // are never candidates); ids are spread as contiguous runs of `per`
  const double* W = a.W + ((long long)b * a.Hkv + g) * a.MB;
  const int per = (a.MB + 255) / 256;  // ids per thread, <= PT
  const int j0 = tid * per;
  double wv[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) wv[i] = (i < per && j0 + i < a.MB) ? W[j0 + i] : 0.0;
  if (nb <= k) {  // every block, then padding
    for (int i = tid; i < k; i += 256) out[i] = i < nb ? i : -1;
    return;
  }
  const int R = a.recent;  // newest blocks always kept
  const int M = k - 1 - R;  // free picks among blocks 1..nb-R-1

  bool cand[PT];
  unsigned hi[PT], lo[PT];
  unsigned hmin = 0xFFFFFFFFu, hmax = 0u;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    cand[i] = i < per && j >= 1 && j < nb - R;
    const unsigned long long key = cand[i] ? order_key(wv[i]) : 0ull;
    hi[i] = (unsigned)(key >> 32);
    lo[i] = (unsigned)key;
    if (cand[i]) {
      hmin = min(hmin, hi[i]);
      hmax = max(hmax, hi[i]);
    }
  }
  // phase 1: threshold on the high 32 bits of the key
  unsigned T_hi = 0u, T_lo = 0u;
  int rem_hi = 0, rem_lo = 0, n_eq = 0;
  bool need_lo = false;
  bool eqh[PT];
  if (M > 0) {
    unsigned mn, mx;
    block_min_max_256(hmin, hmax, mm_tmp, &mn, &mx);
    if (mn == mx) {
      T_hi = mn;
      rem_hi = M;
    } else {
      const int top_bit = 31 - __clz(mn ^ mx);
      radix_select_u32<PT>(hi, cand, M, top_bit / 8, mn, hist, &sh_T, &sh_rem, &T_hi, &rem_hi);
    }
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      eqh[i] = cand[i] && hi[i] == T_hi;
      cnt += eqh[i] ? 1 : 0;
    }
    int tot;
    (void)block_exclusive_scan_256(cnt, scan_tmp, &tot);
    n_eq = tot;
    // phase 2 (only when the threshold bucket holds more keys than needed):
    // threshold on the low 32 bits among the keys tied on the high bits
    need_lo = rem_hi < n_eq;
    if (need_lo) {
      unsigned lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
      for (int i = 0; i < PT; ++i)
        if (eqh[i]) {
          lmin = min(lmin, lo[i]);
          lmax = max(lmax, lo[i]);
        }
      unsigned mn2, mx2;
      block_min_max_256(lmin, lmax, mm_tmp, &mn2, &mx2);
      if (mn2 == mx2) {
        T_lo = mn2;
        rem_lo = rem_hi;
      } else {
        const int top_bit = 31 - __clz(mn2 ^ mx2);
        radix_select_u32<PT>(lo, eqh, rem_hi, top_bit / 8, mn2, hist, &sh_T, &sh_rem, &T_lo, &rem_lo);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PT; ++i) eqh[i] = false;
  }
  // ties on the full key go to the lowest block ids
  int n_tie = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) n_tie += (need_lo && eqh[i] && lo[i] == T_lo) ? 1 : 0;
  int tot;
  int tie_before = block_exclusive_scan_256(n_tie, scan_tmp, &tot);
  int n_sel = 0;
  unsigned chosen = 0u;  // bit i: id j0+i selected
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    if (i >= per || j >= nb) continue;
    bool take;
    if (j == 0 || j >= nb - R) {
      take = true;
    } else if (!cand[i] || M == 0) {
      take = false;
    } else if (hi[i] != T_hi) {
      take = hi[i] > T_hi;
    } else if (!need_lo) {
      take = true;  // the whole bucket is needed
    } else if (lo[i] != T_lo) {
      take = lo[i] > T_lo;
    } else {
      take = tie_before < rem_lo;
      ++tie_before;
    }
    if (take) {
      chosen |= 1u << i;
      ++n_sel;
    }
  }
  int pos = block_exclusive_scan_256(n_sel, scan_tmp, &tot);
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if ((chosen & (1u << i)) && pos < k) out[pos++] = j0 + i;
  for (int i = tot + tid; i < k; i += 256) out[i] = -1;
}

template <int QK, int SK, int D, int G>
void launch_bounds_one(const BoundArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.MB + kBoundBlocks - 1) / kBoundBlocks + (a.append == 1 ? 1 : 0)), (unsigned)a.Hkv,
                  (unsigned)a.B);
  hipLaunchKernelGGL((bounds_kernel<QK, SK, D, G>), grid, dim3(64 * bound_waves<G, SK>()), 0, s, a);
}

template <int QK, int SK, int D>
hipError_t launch_bounds_g(const BoundArgs& a, int G, hipStream_t s) {
  switch (G) {
    case 1: launch_bounds_one<QK, SK, D, 1>(a, s); break;
    case 2: launch_bounds_one<QK, SK, D, 2>(a, s); break;
    case 4: launch_bounds_one<QK, SK, D, 4>(a, s); break;
    case 8: launch_bounds_one<QK, SK, D, 8>(a, s); break;
    default: launch_bounds_one<QK, SK, D, 16>(a, s); break;
  }
  return hipGetLastError();
}

template <int QK, int SK>
hipError_t launch_bounds_d(const BoundArgs& a, int G, hipStream_t s) {
  return a.D == 64 ? launch_bounds_g<QK, SK, 64>(a, G, s) : launch_bounds_g<QK, SK, 128>(a, G, s);
}

}  // namespace

hipError_t launch_bounds(const BoundArgs& a, int q_kind, int summ_kind, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  if (q_kind == K_F32 && summ_kind == K_F32) return launch_bounds_d<K_F32, K_F32>(a, G, s);
  if (q_kind == K_BF16 && summ_kind == K_BF16) return launch_bounds_d<K_BF16, K_BF16>(a, G, s);
  return launch_bounds_d<K_BF16, K_F32>(a, G, s);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const dim3 grid((unsigned)a.Hkv, (unsigned)a.B);
  const int per = (a.MB + 255) / 256;
  if (per <= 2)
    hipLaunchKernelGGL((topk_kernel<2>), grid, dim3(256), 0, s, a);
  else if (per <= 8)
    hipLaunchKernelGGL((topk_kernel<8>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((topk_kernel<32>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvs
