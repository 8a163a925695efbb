// kvs_append.h -- appending one decode token of one (sequence, KV head)
// unit (page "KV 稀疏化", §7 "HiSparse": the newest KV is written to the
// device cache, and KV that is no longer being written sinks to the host
// tier).  Shared by the append kernel and by the scoring kernels, which run
// it beside their scoring work (the exact bounds kernel in each unit's first
// workgroup, the matrix-core one in one more workgroup per unit).
//
// For len = seq_lens[b] > 0 the token t = len-1 lands in block j = t/S, slot
// s = t%S of page block_table[b][j]: thread c writes channel c of K (row s of
// the token-major tile) and of V (column s%T of run s/T), and folds the K
// value into the block's summary -- min/max with the stored summary, or the
// value itself when s = 0 opens the block.  The stored summary must already
// cover tokens jS..t-1 (as kvs_build_summaries or earlier appends leave it).
// When the token fills the block (len % S == 0) the block is sealed: after a
// workgroup barrier its K and V tiles (and fp8 scales) are copied with
// 16-byte vectors to the host tier, byte for byte.
#pragma once

#include "kvs_internal.h"

namespace kvs {

template <int KVK>
struct ElemT;
template <>
struct ElemT<K_F32> {
  using T = uint32_t;
};
template <>
struct ElemT<K_BF16> {
  using T = uint16_t;
};
template <>
struct ElemT<K_FP8> {
  using T = uint8_t;
};

// Every thread of the NT-thread workgroup calls it (D <= NT); all exits are
// uniform over the workgroup.
template <int KVK, int D, int NT>
__device__ __forceinline__ void append_token_unit(const AppendArgs& a, int b, int g) {
  static_assert(D <= NT, "one thread per channel");
  using E = typename ElemT<KVK>::T;
  constexpr int EB = elem_bytes<KVK>();
  const int tid = threadIdx.x;
  const long long unit = (long long)b * a.Hkv + g;
  const int groups = KVK == K_FP8 ? D / a.qg : 0;
  const int c = tid < D ? tid : D - 1;  // threads past D only help with the seal copy
  // loads that need no length go out with the length itself
  const int len = a.seq_lens[b];
  const E kv = static_cast<const E*>(a.k_new)[unit * D + c];
  const E vv = static_cast<const E*>(a.v_new)[unit * D + c];
  float ksc = 1.0f;
  if constexpr (KVK == K_FP8) ksc = a.k_new_scales[unit * groups + c / a.qg];
  if (len < 0 || len > a.MB * a.S) {
    if (tid == 0 && g == 0) raise_flag(a.err, 0x1u);
    return;
  }
  if (len == 0) return;
  const int S = a.S, T = S < 32 ? S : 32;
  const int t = len - 1, j = t / S, s = t % S;
  const int page = a.block_table[(long long)b * a.MB + j];
  // the block's stored summary (its tokens before t) is read beside the page
  const long long row = (unit * a.MB + j) * 2 * D;  // min at [0, D), max at [D, 2D)
  float old_mn = 0.0f, old_mx = 0.0f;
  if (s > 0 && !a.skip_summary) {
    if constexpr (KVK == K_BF16) {
      const uint16_t* ps = static_cast<const uint16_t*>(a.summ) + row;
      old_mn = bf16_lo(ps[c]);
      old_mx = bf16_lo(ps[D + c]);
    } else {
      const float* ps = static_cast<const float*>(a.summ) + row;
      old_mn = ps[c];
      old_mx = ps[D + c];
    }
  }
  if (page < 0 || page >= a.P) {
    if (tid == 0) raise_flag(a.err, 0x2u);
    return;
  }
  const long long tile = (long long)page * a.Hkv + g;  // (page, head) tile
  if (tid < D) {
    static_cast<E*>(a.k_pool)[(tile * S + s) * D + c] = kv;
    static_cast<E*>(a.v_pool)[((tile * (S / T) + s / T) * D + c) * T + s % T] = vv;
  }
  if (tid < D && !a.skip_summary) {
    float x;  // the K element's value, as the summaries and attention read it
    if constexpr (KVK == K_F32) {
      x = __uint_as_float(kv);
    } else if constexpr (KVK == K_BF16) {
      x = bf16_lo((uint32_t)kv);
    } else {
      float f[4];
      fp8x4_to_f32((uint32_t)kv, f);
      x = f[0] * ksc;
    }
    const float mn = s > 0 ? fminf(old_mn, x) : x;
    const float mx = s > 0 ? fmaxf(old_mx, x) : x;
    if constexpr (KVK == K_BF16) {
      uint16_t* ps = static_cast<uint16_t*>(a.summ) + row;
      ps[c] = (uint16_t)bf16_bits_exact(mn);
      ps[D + c] = (uint16_t)bf16_bits_exact(mx);
    } else {
      float* ps = static_cast<float*>(a.summ) + row;
      ps[c] = mn;
      ps[D + c] = mx;
    }
  }
  if constexpr (KVK == K_FP8) {
    if (tid < groups) {
      a.k_scales[(tile * S + s) * groups + tid] = a.k_new_scales[unit * groups + tid];
      a.v_scales[(tile * S + s) * groups + tid] = a.v_new_scales[unit * groups + tid];
    }
  }
  if (!a.host_k || len % S != 0) return;
  // the block is full: seal it into the host tier once every thread's writes
  // of this token are visible to the workgroup
  __syncthreads();
  const long long tile_bytes = (long long)S * D * EB;
  const long long host_tile = unit * a.MB + j;
  const u32x4* sk = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.k_pool) + tile * tile_bytes);
  const u32x4* sv = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v_pool) + tile * tile_bytes);
  u32x4* dk = reinterpret_cast<u32x4*>(static_cast<char*>(a.host_k) + host_tile * tile_bytes);
  u32x4* dv = reinterpret_cast<u32x4*>(static_cast<char*>(a.host_v) + host_tile * tile_bytes);
  const int nvec = (int)(tile_bytes / 16);
  for (int i = tid; i < nvec; i += NT) {
    const u32x4 x = sk[i];
    const u32x4 y = sv[i];
    dk[i] = x;
    dv[i] = y;
  }
  if constexpr (KVK == K_FP8) {
    const long long ns = (long long)S * groups;
    for (int i = tid; i < ns; i += NT) {
      a.host_ks[host_tile * ns + i] = a.k_scales[tile * ns + i];
      a.host_vs[host_tile * ns + i] = a.v_scales[tile * ns + i];
    }
  }
}

}  // namespace kvs
