// kvs_append.hip -- the decode-token append as a launch of its own: one
// 256-thread workgroup per (sequence, KV head) unit runs append_token_unit
// (kvs_append.h).  Roofline: a few hundred bytes per unit (K and V of one
// token, one summary row), plus 2*S*D*elem bytes over the host link for a
// unit whose block has just filled; launch latency dominates.
#include "kvs_append.h"

namespace kvs {
namespace {

constexpr int kAppendThreads = 256;

template <int KVK, int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  append_token_unit<KVK, D, kAppendThreads>(a, blockIdx.y, blockIdx.x);
}

template <int KVK>
void launch_kind(const AppendArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.Hkv, (unsigned)a.B);
  if (a.D == 64)
    hipLaunchKernelGGL((append_kernel<KVK, 64>), grid, dim3(kAppendThreads), 0, s, a);
  else
    hipLaunchKernelGGL((append_kernel<KVK, 128>), grid, dim3(kAppendThreads), 0, s, a);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int kv_kind, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (kv_kind == K_F32)
    launch_kind<K_F32>(a, s);
  else if (kv_kind == K_BF16)
    launch_kind<K_BF16>(a, s);
  else
    launch_kind<K_FP8>(a, s);
  return hipGetLastError();
}

}  // namespace kvs
