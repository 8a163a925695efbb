// kvs_select.hip -- query-aware block scores and top-k selection (page
// "KV 稀疏化", §5 "Quest": coarse-filter the blocks with the query and the
// summaries, keep the top-k; the sink block and the newest block are always
// kept, same page §2 and "SparDA：把KV選擇提前一層…" §4.2).
//
// bounds_kernel: one thread per (block, query head).  The block score is
// U = sum_c max(q_c*mn_c, q_c*mx_c); since mx_c >= mn_c the larger product is
// q_c*mx_c when q_c >= 0 and q_c*mn_c otherwise, so each channel costs one
// select and one fp64 fma.  Every product of a bf16/fp32 query with a
// bf16/fp32 summary is exact in fp64, and the sum runs in ascending c, so
// the result is bit-identical to the plain ordered fp64 sum; the max over a
// group's G heads is taken across G adjacent lanes.  Roofline: HBM-bound read
// of the summaries (2*D*elem bytes per block and KV head).
//
// topk_kernel: one 256-thread workgroup per (sequence, KV head).  Scores are
// mapped to order-preserving 64-bit keys and a most-significant-digit radix
// select (8 passes of 8 bits, LDS histogram) finds the (k-2)-th largest key
// among blocks 1..nb-2; ties at that key go to the lowest block ids, the
// (W desc, id asc) order.  A block-wide prefix sum then writes the chosen
// ids in ascending order.  Latency-bound.
#include "kvs_internal.h"

namespace kvs {
namespace {

template <int QK, int SK, int D, int G>
__global__ __launch_bounds__(256) void bounds_kernel(BoundArgs a) {
  constexpr int NBLK = 256 / G;  // blocks per workgroup
  constexpr int QPAD = 4;
  constexpr int SVEC = Vec16<SK>::N;
  __shared__ float qs[G][D + QPAD];
  const int b = blockIdx.z, g = blockIdx.y;
  const int tid = threadIdx.x;
  // stage the group's G query rows (exact in fp32 for bf16/fp32 queries)
  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, c = i % D;
    const long long qi = ((long long)b * a.Hq + (long long)g * G + h) * D + c;
    float v;
    if constexpr (QK == K_F32)
      v = static_cast<const float*>(a.q)[qi];
    else
      v = __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.q)[qi] << 16);
    qs[h][c] = v;
  }
  __syncthreads();

  const int h = tid % G;
  const int j = blockIdx.x * NBLK + tid / G;
  int len = a.seq_lens[b];
  const int cap = a.MB * a.S;
  if (len < 0 || len > cap) {
    if (tid == 0 && blockIdx.x == 0 && g == 0) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  const int nb = (len + a.S - 1) / a.S;

  double acc = -__builtin_inf();
  if (j < nb) {
    acc = 0.0;
    const char* sb = static_cast<const char*>(a.summ);
    const long long row = (((long long)b * a.Hkv + g) * a.MB + j) * 2 * D;
    const char* pmn = sb + row * elem_bytes<SK>();
    const char* pmx = sb + (row + D) * elem_bytes<SK>();
#pragma unroll 2
    for (int c0 = 0; c0 < D; c0 += SVEC) {
      float mn[SVEC], mx[SVEC];
      Vec16<SK>::load(pmn + c0 * elem_bytes<SK>(), mn);
      Vec16<SK>::load(pmx + c0 * elem_bytes<SK>(), mx);
#pragma unroll
      for (int e = 0; e < SVEC; ++e) {
        const float qc = qs[h][c0 + e];
        const float x = qc >= 0.0f ? mx[e] : mn[e];
        acc = __builtin_fma((double)qc, (double)x, acc);
      }
    }
  }
  double w = acc;
#pragma unroll
  for (int off = 1; off < G; off <<= 1) {
    const double o = __shfl_xor(w, off);
    w = o > w ? o : w;
  }
  if (h == 0 && j < a.MB) {
    const long long wi = ((long long)b * a.Hkv + g) * a.MB + j;
    a.W[wi] = w;
    if (a.bounds_out) a.bounds_out[wi] = w;
  }
}

// order-preserving map of a double (no NaN) to uint64; -0 and +0 coincide
__device__ __forceinline__ unsigned long long order_key(double w) {
  const double z = w + 0.0;  // -0 -> +0
  const unsigned long long u = (unsigned long long)__double_as_longlong(z);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

template <int PT>  // candidates per thread (contiguous block ids)
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ unsigned int hist[256];
  __shared__ int scan_tmp[4];
  __shared__ unsigned long long sh_prefix;
  __shared__ int sh_rem;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int k = a.k;
  int len = a.seq_lens[b];
  const int cap = a.MB * a.S;
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int nb = (len + a.S - 1) / a.S;
  int32_t* out = a.sel + ((long long)b * a.Hkv + g) * k;

  if (nb <= k) {  // every block, then padding
    for (int i = tid; i < k; i += 256) out[i] = i < nb ? i : -1;
    return;
  }
  const int M = k - 2;  // free picks among blocks 1..nb-2
  const double* W = a.W + ((long long)b * a.Hkv + g) * a.MB;
  const int per = (nb + 255) / 256;  // ids per thread, <= PT
  const int j0 = tid * per;

  unsigned long long key[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    const bool cand = i < per && j >= 1 && j <= nb - 2;
    key[i] = cand ? order_key(W[j]) : 0ull;
  }

  unsigned long long prefix = 0ull, mask = 0ull;
  int rem = M;  // rank (1-based, from the top) still to locate
  if (M > 0) {
    for (int pass = 7; pass >= 0; --pass) {
      const int shift = pass * 8;
      hist[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int j = j0 + i;
        const bool cand = i < per && j >= 1 && j <= nb - 2;
        if (cand && (key[i] & mask) == prefix)
          atomicAdd(&hist[(unsigned)(key[i] >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns digits 255-4l .. 252-4l (highest digits first)
        unsigned int c4[4], s = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c4[e] = hist[255 - 4 * tid - e];
          s += c4[e];
        }
        unsigned int incl = s;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const unsigned int o = __shfl_up(incl, off);
          if (tid >= off) incl += o;
        }
        unsigned int above = incl - s;  // count in higher digits
        if ((int)above < rem && rem <= (int)incl) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if ((int)(above + c4[e]) >= rem) {
              sh_prefix = prefix | ((unsigned long long)(255 - 4 * tid - e) << shift);
              sh_rem = rem - (int)above;
              break;
            }
            above += c4[e];
          }
        }
      }
      __syncthreads();
      prefix = sh_prefix;
      rem = sh_rem;
      mask |= 0xFFull << shift;
      __syncthreads();
    }
  }
  // prefix = the M-th largest key T; rem = how many keys equal to T to take
  int n_eq = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    const bool cand = i < per && j >= 1 && j <= nb - 2;
    n_eq += (M > 0 && cand && key[i] == prefix) ? 1 : 0;
  }
  int tot;
  int eq_before = block_exclusive_scan_256(n_eq, scan_tmp, &tot);
  int n_sel = 0;
  unsigned int chosen = 0u;  // bit i: id j0+i selected
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    if (i >= per || j >= nb) continue;
    bool take;
    if (j == 0 || j == nb - 1) {
      take = true;
    } else if (M == 0) {
      take = false;
    } else if (key[i] > prefix) {
      take = true;
    } else if (key[i] == prefix) {
      take = eq_before < rem;
      ++eq_before;
    } else {
      take = false;
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

template <int QK, int SK, int D>
hipError_t launch_bounds_g(const BoundArgs& a, int G, hipStream_t s) {
  const int nblk = 256 / G;
  const dim3 grid((unsigned)((a.MB + nblk - 1) / nblk), (unsigned)a.Hkv, (unsigned)a.B);
  switch (G) {
    case 1: hipLaunchKernelGGL((bounds_kernel<QK, SK, D, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((bounds_kernel<QK, SK, D, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((bounds_kernel<QK, SK, D, 4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((bounds_kernel<QK, SK, D, 8>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((bounds_kernel<QK, SK, D, 16>), grid, dim3(256), 0, s, a); break;
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
