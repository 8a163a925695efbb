// kvs_summaries.hip -- per-block channel-wise min/max of K (the block
// summary of page "KV 稀疏化", §5 "Quest").
//
// One wavefront per (sequence, KV head, block).  Lanes read the block's K
// tile in coalesced 16-byte vectors (LPR lanes cover one token row of D
// channels, RPI rows per wave-instruction), keep a running min/max per
// channel in registers, then fold the RPI row groups with cross-lane
// shuffles.  fp8 codes are decoded and multiplied by their group scale in
// fp32 before the comparison, the same value attention uses.
//
// Roofline: HBM-bound streaming read of S*D*elem bytes (+ fp8 scales) per
// block and 2*D*out_elem bytes written; no arithmetic to speak of.
#include "kvs_internal.h"

namespace kvs {
namespace {

template <int KVK, int D>
__global__ __launch_bounds__(256) void summaries_kernel(SummArgs a) {
  constexpr int VEC = Vec16<KVK>::N;  // elements per 16-byte load
  constexpr int LPR = D / VEC;        // lanes per token row
  constexpr int RPI = kWave / LPR;    // rows per wave-instruction
  static_assert(LPR >= 1 && LPR <= kWave && (kWave % LPR) == 0, "bad row split");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.z, g = blockIdx.y;
  const int S = a.S;

  int len = a.seq_lens[b];
  const int cap = a.MB * S;
  if (len < 0 || len > cap) {
    if (lane == 0 && wave == 0 && blockIdx.x == 0 && g == 0) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  const int nb = (len + S - 1) / S;
  int first = a.first_block ? a.first_block[b] : 0;
  if (first < 0) first = 0;
  const long long end_ll = (long long)first + a.num_rebuild;
  const int end = end_ll < nb ? (int)end_ll : nb;
  const long long jl = (long long)first + (long long)blockIdx.x * 4 + wave;
  if (jl >= end) return;
  const int j = (int)jl;

  const int page = a.block_table[(long long)b * a.MB + j];
  if (page < 0 || page >= a.P) {
    if (lane == 0) raise_flag(a.err, 0x2u);
    return;
  }
  const int ntok = min(S, len - j * S);
  const long long tile = ((long long)page * a.Hkv + g) * S;  // first token row
  const int col = (lane % LPR) * VEC;
  const int r0 = lane / LPR;

  float mn[VEC], mx[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
  const char* base = static_cast<const char*>(a.k_pool);
  for (int t = r0; t < ntok; t += RPI) {
    float v[VEC];
    Vec16<KVK>::load(base + ((tile + t) * D + col) * elem_bytes<KVK>(), v);
    if constexpr (KVK == K_FP8) {
      const int groups = D / a.qg;
      const float sc = a.k_scales[(tile + t) * groups + col / a.qg];
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = v[e] * sc;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      mn[e] = fminf(mn[e], v[e]);
      mx[e] = fmaxf(mx[e], v[e]);
    }
  }
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      mn[e] = fminf(mn[e], __shfl_xor(mn[e], off));
      mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], off));
    }
  }
  if (lane >= LPR) return;
  const long long orow = (((long long)b * a.Hkv + g) * a.MB + j) * 2 * D;
  if constexpr (KVK == K_BF16) {
    uint16_t* o = static_cast<uint16_t*>(a.out) + orow;
    uint4 wmn, wmx;
    uint32_t* pm = reinterpret_cast<uint32_t*>(&wmn);
    uint32_t* px = reinterpret_cast<uint32_t*>(&wmx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pm[i] = bf16_bits_exact(mn[2 * i]) | (bf16_bits_exact(mn[2 * i + 1]) << 16);
      px[i] = bf16_bits_exact(mx[2 * i]) | (bf16_bits_exact(mx[2 * i + 1]) << 16);
    }
    *reinterpret_cast<uint4*>(o + col) = wmn;
    *reinterpret_cast<uint4*>(o + D + col) = wmx;
  } else {
    float* o = static_cast<float*>(a.out) + orow;
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      *reinterpret_cast<float4*>(o + col + e) = make_float4(mn[e], mn[e + 1], mn[e + 2], mn[e + 3]);
      *reinterpret_cast<float4*>(o + D + col + e) = make_float4(mx[e], mx[e + 1], mx[e + 2], mx[e + 3]);
    }
  }
}

template <int KVK>
hipError_t launch_d(const SummArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.num_rebuild + 3) / 4), (unsigned)a.Hkv, (unsigned)a.B);
  if (a.D == 64)
    hipLaunchKernelGGL((summaries_kernel<KVK, 64>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((summaries_kernel<KVK, 128>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
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
