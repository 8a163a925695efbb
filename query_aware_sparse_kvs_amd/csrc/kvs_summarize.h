// kvs_summarize.h -- the summary of one block (per channel: min and max of
// K over the block's valid tokens; page "KV 稀疏化", §5 "Quest"), computed by
// one workgroup (256 threads unless the caller's kernel has more).  Shared by the summaries kernel and by the
// scoring kernels, whose extra workgroups rebuild each sequence's newest
// block while the others score.
//
// The K tile (S rows x D channels) is read as 16-byte vectors, every load of
// a thread issued before any comparison; a thread always sees the same
// channel chunk (the vectors of a row are spread over LPR threads), so it
// folds its rows in registers, then the row groups are folded by cross-lane
// shuffles and the four wavefronts through LDS.  fp8 codes are decoded and
// multiplied by their group scale in fp32 first, the same value attention
// uses.
#pragma once

#include "kvs_internal.h"

namespace kvs {

// Block j of (sequence b, KV head g), len = that sequence's clamped length,
// j < ceil(len / S).  Every thread of the NT-thread workgroup must call it;
// `red` is kSummRed<D, NT> floats of the caller's LDS, free for this call.
template <int D, int NT = 256>
constexpr int kSummRed = 2 * D * (NT / 64);

template <int KVK, int D, int S, int NT = 256>
__device__ __forceinline__ void summarize_block(const SummArgs& a, int b, int g, int j, int len, float* red) {
  constexpr int VEC = Vec16<KVK>::N;              // elements per 16-byte vector
  constexpr int LPR = D / VEC;                    // vectors per token row
  constexpr int NV = S * LPR;                     // vectors per tile
  constexpr int NPT = (NV + NT - 1) / NT;         // vectors per thread
  constexpr int RSTEP = NT / LPR;                 // row stride between a thread's vectors
  constexpr int NW = NT / kWave;
  static_assert(NT % LPR == 0 && LPR <= kWave, "row split must divide the workgroup");
  static_assert(NW * 2 * LPR * VEC == kSummRed<D, NT>, "reduction buffer size");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int page = a.block_table[(long long)b * a.MB + j];
  if (page < 0 || page >= a.P) {
    if (tid == 0) raise_flag(a.err, 0x2u);
    return;
  }
  const int ntok = min(S, len - j * S);
  const long long tile = ((long long)page * a.Hkv + g) * S;  // first token row
  const int col = (tid % LPR) * VEC;
  const int r0 = tid / LPR;
  const char* base = static_cast<const char*>(a.k_pool);

  uint4 raw[NPT];
#pragma unroll
  for (int x = 0; x < NPT; ++x) {
    const int row = r0 + x * RSTEP;
    if (row < ntok) raw[x] = *reinterpret_cast<const uint4*>(base + ((tile + row) * D + col) * elem_bytes<KVK>());
  }
  float sc[NPT];
  if constexpr (KVK == K_FP8) {
    const int groups = D / a.qg;
#pragma unroll
    for (int x = 0; x < NPT; ++x) {
      const int row = r0 + x * RSTEP;
      sc[x] = row < ntok ? a.k_scales[(tile + row) * groups + col / a.qg] : 1.0f;
    }
  }
  float mn[VEC], mx[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
#pragma unroll
  for (int x = 0; x < NPT; ++x) {
    const int row = r0 + x * RSTEP;
    if (row >= ntok) continue;
    float v[VEC];
    const uint32_t ws[4] = {raw[x].x, raw[x].y, raw[x].z, raw[x].w};
    if constexpr (KVK == K_F32) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(ws[e]);
    } else if constexpr (KVK == K_BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16_lo(ws[e]);
        v[2 * e + 1] = bf16_hi(ws[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) fp8x4_to_f32(ws[e], v + 4 * e);
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = v[e] * sc[x];
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      mn[e] = fminf(mn[e], v[e]);
      mx[e] = fmaxf(mx[e], v[e]);
    }
  }
  // fold the row groups inside the wavefront, then across wavefronts
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      mn[e] = fminf(mn[e], __shfl_xor(mn[e], off));
      mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], off));
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      red[((wave * 2 + 0) * LPR + lane) * VEC + e] = mn[e];
      red[((wave * 2 + 1) * LPR + lane) * VEC + e] = mx[e];
    }
  }
  __syncthreads();
  if (wave != 0 || lane >= LPR) return;
#pragma unroll
  for (int w = 1; w < NW; ++w)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      mn[e] = fminf(mn[e], red[((w * 2 + 0) * LPR + lane) * VEC + e]);
      mx[e] = fmaxf(mx[e], red[((w * 2 + 1) * LPR + lane) * VEC + e]);
    }
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

// The summary of sequence b's newest block (nb - 1) for KV head g, from a
// workgroup of a kernel launched for other work (uniform early role); `red`
// as for summarize_block.
template <int KVK, int D, int NT = 256>
__device__ __forceinline__ void rebuild_newest_summary(const SummArgs& a, int b, int g, float* red) {
  int len = a.seq_lens[b];
  const int cap = a.MB * a.S;
  len = len < 0 ? 0 : (len > cap ? cap : len);  // the scoring kernels flag bad lengths
  const int nb = (len + a.S - 1) / a.S;
  if (nb == 0) return;
  switch (a.S) {
    case 16: summarize_block<KVK, D, 16, NT>(a, b, g, nb - 1, len, red); break;
    case 32: summarize_block<KVK, D, 32, NT>(a, b, g, nb - 1, len, red); break;
    default: summarize_block<KVK, D, 64, NT>(a, b, g, nb - 1, len, red); break;
  }
}

}  // namespace kvs
