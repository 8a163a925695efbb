// kvs_select.hip -- query-aware block scores and top-k selection (page
// "KV 稀疏化", §5 "Quest": coarse-filter the blocks with the query and the
// summaries, keep the top-k; the sink block and the newest block are always
// kept, same page §2 and "SparDA：把KV選擇提前一層…" §4.2).
//
// bounds_kernel: a workgroup of 4 wavefronts (8 for groups of 8 or more
// query heads, one per head) stages 64 consecutive blocks' summaries in LDS
// with coalesced 16-byte loads, in two channel halves so that the first
// half's sums run while the second half arrives; lane = block, wavefront w takes query heads
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
// topk_kernel: one 256-thread workgroup per (sequence, KV head) runs the
// selection of kvs_topk.h.  Latency-bound.
//
// With score smoothing on, the bounds kernel ranks blocks by the smoothed
// score alpha*W + (1-alpha)*history ("SparDA…" §6.1) instead of W itself.
// With accumulation on, it adds the (smoothed) score to the sum of earlier
// layers' scores already in the output ("SparDA…" §3.1, §4.1: a few shallow
// layers' scores fused into one mask for the deeper layers).
#include "kvs_append.h"
#include "kvs_summarize.h"
#include "kvs_topk.h"

namespace kvs {
namespace {

constexpr int kBoundBlocks = 64;  // blocks per bounds workgroup (lane = block)

// wavefronts per bounds workgroup: one per query head of the group, 4 to 8.
// With fp32 summaries the 64-block chunk takes about 77 KB of LDS, so two
// workgroups (16 wavefronts) still share a compute unit; more wavefronts per
// workgroup hide more of the dependent fp64 chain's latency.
template <int G, int SK>
constexpr int bound_waves() {
  return G >= 8 ? 8 : 4;
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
  constexpr int EB = SK == K_BF16 ? 2 : 4;   // summary element bytes
  constexpr int ROWB = (SK == K_MEAN ? 1 : 2) * D * EB;  // bytes of one block's summary
  constexpr int ROWP = ROWB + 16;            // padded LDS row (bank spread)
  constexpr int NV = NB * ROWB / 16;         // 16-byte vectors of the chunk
  constexpr int NPT = NV / NT;
  static_assert(NV % NT == 0, "whole vectors per thread");
  constexpr int VEC = 16 / EB;               // summary elements per 16 bytes
  constexpr int SEGS = SK == K_MEAN ? 1 : 2;  // rows per block: min and max, or the mean
  constexpr int SEGV = D * EB / 32;           // 16-byte vectors of half a row
  constexpr int VPH = SEGS * SEGV;            // vectors of one block's channel half
  constexpr int NPH = NPT / 2;                // vectors per thread and half
  static_assert(NPT % 2 == 0 && (D / 2) % VEC == 0, "whole vectors per half");
  // byte offset in a block's row of vector w (< VPH) of channel half `half`
  auto half_offset = [](int half, int w) { return (w / SEGV) * (D * EB) + half * (D * EB / 2) + (w % SEGV) * 16; };
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
  // the sequence length as a scalar load (no kernel writes it), in flight
  // beside the vector loads below instead of queued behind them
  int len = *(const __attribute__((address_space(4))) int32_t*)(a.seq_lens + b);

  // the query first: loads complete in issue order, so the query must not
  // queue behind the chunk
  constexpr int QPT = (G * D + NT - 1) / NT;
  uint32_t qv[QPT];  // raw bits: converted only after the chunk's loads are out
#pragma unroll
  for (int y = 0; y < QPT; ++y) {
    // unconditional loads (index clamped) keep the load counter exact
    const int i = min(y * NT + tid, G * D - 1);
    const int h = i / D, c = i % D;
    const long long qi = ((long long)b * a.Hq + (long long)g * G + h) * D + c;
    if constexpr (QK == K_F32)
      qv[y] = static_cast<const uint32_t*>(a.q)[qi];
    else
      qv[y] = static_cast<const uint16_t*>(a.q)[qi];
  }
  __builtin_amdgcn_sched_barrier(0);  // the query loads stay ahead of the chunk's
  // stage the chunk's summaries in two channel halves (channels [0, D/2),
  // then [D/2, D), of the min and the max rows of all NB blocks), every load
  // issued before any use and not waiting for seq_lens (blocks past nb are
  // read but never used): the first half's fp64 chains run while the
  // second half is still arriving
  const char* src = static_cast<const char*>(a.summ) + (((long long)b * a.Hkv + g) * a.MB + j0) * ROWB;
  u32x4 raw[NPT];
#pragma unroll
  for (int x = 0; x < NPT; ++x) {
    if (x == NPH) __builtin_amdgcn_sched_barrier(0);  // the first half's loads go out first
    const int half = x / NPH, u = (x % NPH) * NT + tid;
    // blocks past the array read its last block of the chunk instead (their
    // rows are never used): no branch, so the load counter stays exact and
    // the first half waits for its own loads only
    const int blk = min(u / VPH, nmem - 1), off = half_offset(half, u % VPH);
    raw[x] = *reinterpret_cast<const u32x4*>(src + (long long)blk * ROWB + off);
  }
  __builtin_amdgcn_sched_barrier(0);
  // each unit's first workgroup also appends the decode token (a workgroup
  // of its own would leave some compute units with two scoring workgroups;
  // mean tables are rebuilt instead).  Its loads go out behind the chunk's,
  // its block's page and stored summary once the length is in, and its
  // stores after the scores, so the append never holds up the chunk.  Every
  // workgroup issues the same loads (the others read a spare address), so
  // the waits for the chunk stay exact.
  const bool appender = SK != K_MEAN && a.append == 2 && blockIdx.x == 0;  // uniform
  const int tkind = SK == K_BF16 ? (int)K_BF16 : (a.app_kv == K_FP8 ? (int)K_FP8 : (int)K_F32);  // K storage
  const int32_t* spare = a.seq_lens;
  TokenIn tin{0u, 0u, 1.0f, 0};
  if constexpr (SK == K_BF16)
    tin = load_token_in<K_BF16, D, true>(a.tok, b, g, appender, spare);
  else if constexpr (SK == K_F32)
    tin = load_token_in_word<D>(a.tok, b, g, appender, tkind == K_FP8, spare);
  // the query as fp64, and per head the words' choice of max (mask bits set) or min
#pragma unroll
  for (int y = 0; y < QPT; ++y) {
    const int i = y * NT + tid;
    if (i < G * D) qd[i / D][i % D] = (double)__uint_as_float(QK == K_F32 ? qv[y] : qv[y] << 16);
  }
  const int tok_len = len;
  const int cap = a.MB * a.S;
  if (len < 0 || len > cap) {
    if (tid == 0 && blockIdx.x == 0 && g == 0) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  // the token's block (an invalid length is flagged and appends nothing; an
  // empty sequence appends nothing)
  const bool tok_ok = appender && tok_len >= 1 && tok_len <= a.tok.MB * a.tok.S;
  if (appender && (tok_len < 0 || tok_len > a.tok.MB * a.tok.S) && tid == 0 && g == 0) raise_flag(a.tok.err, 0x1u);
  TokenBlock tblk{0, 0u, 0u};
  if constexpr (SK == K_BF16) {
    tblk = load_token_block<K_BF16, D, true, true>(a.tok, b, g, tok_len, tok_ok, spare);
  } else if constexpr (SK == K_F32) {  // fp8 and fp32 K both keep fp32 summaries
    tblk = load_token_block<K_F32, D, true, true>(a.tok, b, g, tok_len, tok_ok, spare);
  }
  const int nb = (len + a.S - 1) / a.S;
  // one half of the chunk -> its LDS rows
  auto stage_half = [&](int half) {
#pragma unroll
    for (int x = half * NPH; x < half * NPH + NPH; ++x) {
      const int u = (x % NPH) * NT + tid;
      const int blk = u / VPH;
      if (blk < nmem) *reinterpret_cast<u32x4*>(sm + blk * ROWP + half_offset(half, u % VPH)) = raw[x];
    }
  };
  stage_half(0);
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
  for (int half = 0; half < 2; ++half) {
    if (half == 1) {
      stage_half(1);
      __syncthreads();
    }
    if (wave >= G) continue;
    // VEC-channel steps; each step's LDS reads (the lane's min and max
    // words, the heads' masks and fp64 query values) are issued one step
    // ahead of its arithmetic, and the heads' chains are interleaved channel
    // by channel, each still summed in ascending c
    constexpr int NSTEP = (D / 2) / VEC;
    struct Step {
      u32x4 mn, mx, m[HPW];
      double q[HPW][VEC];
    };
    auto load = [&](int st, Step& t) {
      const int c0 = half * (D / 2) + st * VEC;
      t.mn = *reinterpret_cast<const u32x4*>(pmn + c0 * EB);
      t.mx = t.mn;
      if constexpr (SK != K_MEAN) t.mx = *reinterpret_cast<const u32x4*>(pmx + c0 * EB);
#pragma unroll
      for (int i = 0; i < HPW; ++i) {
        const int h = min(wave + NWB * i, G - 1);  // (heads past G: never used)
        if constexpr (SK != K_MEAN) t.m[i] = *reinterpret_cast<const u32x4*>(&qm[h][c0 * EB / 4]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) t.q[i][e] = qd[h][c0 + e];
      }
    };
    Step cur, nxt;
    load(0, cur);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + 1 < NSTEP) load(st + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);  // the next step's reads go out before this step's arithmetic
      float xf[HPW][VEC];
#pragma unroll
      for (int i = 0; i < HPW; ++i) {
        // score q.mean: the row is the mean itself; else the word-wise choice of max or min
        const u32x4 x = SK == K_MEAN ? cur.mn : (cur.mx & cur.m[i]) | (cur.mn & ~cur.m[i]);
        if constexpr (EB == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xf[i][2 * e] = bf16_lo(x[e]);
            xf[i][2 * e + 1] = bf16_hi(x[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) xf[i][e] = __uint_as_float(x[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int i = 0; i < HPW; ++i)
          if (wave + NWB * i < G) acc[i] = __builtin_fma(cur.q[i][e], (double)xf[i][e], acc[i]);
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < NSTEP) cur = nxt;
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
    if (a.accumulate && valid) w = a.W[wi] + w;  // the earlier layers' sum first
    a.W[wi] = w;
  }
  if (tok_ok) {  // the token's stores (and the seal of a block it fills)
    if (tkind == K_BF16)
      store_token<K_BF16, D, NT>(a.tok, b, g, tok_len, tin, tblk);
    else if (tkind == K_FP8)
      store_token<K_FP8, D, NT>(a.tok, b, g, tok_len, tin, tblk);
    else
      store_token<K_F32, D, NT>(a.tok, b, g, tok_len, tin, tblk);
  }
}

template <int PT>  // candidates per thread (contiguous block ids)
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ TopkLds sh;
  const int g = blockIdx.x, b = blockIdx.y;
  const long long unit = (long long)b * a.Hkv + g;
  double wv[PT];
  load_unit_scores<PT>(a.W + unit * a.MB, a.MB, wv);
  int len = a.seq_lens[b];
  const int cap = a.MB * a.S;
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int nb = (len + a.S - 1) / a.S;
  select_unit<PT>(wv, a.MB, nb, a.k, a.recent, a.sel + unit * a.k, sh);
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
  if (summ_kind == K_MEAN)
    return q_kind == K_F32 ? launch_bounds_d<K_F32, K_MEAN>(a, G, s) : launch_bounds_d<K_BF16, K_MEAN>(a, G, s);
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
