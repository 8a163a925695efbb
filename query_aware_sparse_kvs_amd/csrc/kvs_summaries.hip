// kvs_summaries.hip -- per-block channel-wise min/max of K (the block
// summary of page "KV 稀疏化", §5 "Quest"), or its channel-wise mean (the
// same page lists the mean as another summary).
//
// One 256-thread workgroup per (sequence, KV head, block), each running
// summarize_block (kvs_summarize.h).  With `newest` set, the block rebuilt
// is each sequence's last one, nb - 1.
//
// Roofline: HBM-bound streaming read of S*D*elem bytes (+ fp8 scales) per
// block, 2*D*out_elem bytes written; the comparisons are negligible.
#include "kvs_summarize.h"

namespace kvs {
namespace {

template <int KVK, int D, int S>
__global__ __launch_bounds__(256) void summaries_kernel(SummArgs a) {
  __shared__ float red[kSummRed<D>];
  const int tid = threadIdx.x;
  const int b = blockIdx.z, g = blockIdx.y;
  int len = a.seq_lens[b];
  const int cap = a.MB * S;
  if (len < 0 || len > cap) {
    if (tid == 0 && blockIdx.x == 0 && g == 0) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  const int nb = (len + S - 1) / S;
  int first = a.newest ? nb - 1 : (a.first_block ? a.first_block[b] : 0);
  if (first < 0) first = 0;
  const long long end_ll = (long long)first + a.num_rebuild;
  const int end = end_ll < nb ? (int)end_ll : nb;
  const long long jl = (long long)first + blockIdx.x;
  if (jl >= end) return;  // uniform over the workgroup
  const int j = (int)jl;
  summarize_block<KVK, D, S>(a, b, g, j, len, red);
}

// Mean summaries: one thread per channel adds the block's valid tokens in
// ascending order in fp64 (each load of the workgroup reads one token row),
// then stores fp32(sum / n) -- the same rounding steps as the plain
// definition.  Roofline: HBM read of S*D*elem bytes per block.
template <int KVK, int D, int S>
__global__ __launch_bounds__(D) void summaries_mean_kernel(SummArgs a) {
  const int c = threadIdx.x;
  const int b = blockIdx.z, g = blockIdx.y;
  int len = a.seq_lens[b];
  const int cap = a.MB * S;
  if (len < 0 || len > cap) {
    if (c == 0 && blockIdx.x == 0 && g == 0) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  const int nb = (len + S - 1) / S;
  int first = a.newest ? nb - 1 : (a.first_block ? a.first_block[b] : 0);
  if (first < 0) first = 0;
  const long long end_ll = (long long)first + a.num_rebuild;
  const int end = end_ll < nb ? (int)end_ll : nb;
  const long long jl = (long long)first + blockIdx.x;
  if (jl >= end) return;  // uniform over the workgroup
  const int j = (int)jl;
  const int page = a.block_table[(long long)b * a.MB + j];
  if (page < 0 || page >= a.P) {
    if (c == 0) raise_flag(a.err, 0x2u);
    return;
  }
  const int ntok = min(S, len - j * S);
  const long long row0 = ((long long)page * a.Hkv + g) * S;  // first token row of the tile
  float v[S];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    v[t] = 0.0f;
    if (t < ntok) {
      if constexpr (KVK == K_F32) {
        v[t] = static_cast<const float*>(a.k_pool)[(row0 + t) * D + c];
      } else if constexpr (KVK == K_BF16) {
        v[t] = bf16_lo(static_cast<const uint16_t*>(a.k_pool)[(row0 + t) * D + c]);
      } else {
        float f[4];
        fp8x4_to_f32(static_cast<const uint8_t*>(a.k_pool)[(row0 + t) * D + c], f);
        v[t] = f[0] * a.k_scales[(row0 + t) * (D / a.qg) + c / a.qg];
      }
    }
  }
  double sum = 0.0;
#pragma unroll
  for (int t = 0; t < S; ++t)
    if (t < ntok) sum = sum + (double)v[t];
  const double mean = sum / (double)ntok;
  static_cast<float*>(a.out)[(((long long)b * a.Hkv + g) * a.MB + j) * D + c] = (float)mean;
}

template <int KVK, int D>
hipError_t launch_mean(const SummArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.num_rebuild, (unsigned)a.Hkv, (unsigned)a.B);
  switch (a.S) {
    case 16: hipLaunchKernelGGL((summaries_mean_kernel<KVK, D, 16>), grid, dim3(D), 0, s, a); break;
    case 32: hipLaunchKernelGGL((summaries_mean_kernel<KVK, D, 32>), grid, dim3(D), 0, s, a); break;
    default: hipLaunchKernelGGL((summaries_mean_kernel<KVK, D, 64>), grid, dim3(D), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int KVK, int D>
hipError_t launch_s(const SummArgs& a, hipStream_t s) {
  if (a.mean) return launch_mean<KVK, D>(a, s);
  const dim3 grid((unsigned)a.num_rebuild, (unsigned)a.Hkv, (unsigned)a.B);
  switch (a.S) {
    case 16: hipLaunchKernelGGL((summaries_kernel<KVK, D, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((summaries_kernel<KVK, D, 32>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((summaries_kernel<KVK, D, 64>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int KVK>
hipError_t launch_d(const SummArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_s<KVK, 64>(a, s) : launch_s<KVK, 128>(a, s);
}

}  // namespace

hipError_t launch_summaries(const SummArgs& a, int kv_kind, hipStream_t s) {
  if (a.B == 0 || a.num_rebuild == 0) return hipSuccess;
  switch (kv_kind) {
    case K_F32: return launch_d<K_F32>(a, s);
    case K_BF16: return launch_d<K_BF16>(a, s);
    default: return launch_d<K_FP8>(a, s);
  }
}

}  // namespace kvs
