// kvs_summaries.hip -- per-block channel-wise min/max of K (the block
// summary of page "KV 稀疏化", §5 "Quest").
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

template <int KVK, int D>
hipError_t launch_s(const SummArgs& a, hipStream_t s) {
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
