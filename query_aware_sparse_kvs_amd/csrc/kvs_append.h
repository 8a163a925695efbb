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

#include <type_traits>

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

// The append in three phases, so that a caller with loads of its own can
// issue the token's loads first and do the stores last:
//   load_token_in     the token's K and V element of channel c (and its K
//                     group scale), needing no length;
//   load_token_block  for a length len in [1, MB*S]: the page of the token's
//                     block and the block's stored summary of channel c;
//   store_token       the writes, the summary fold and the seal.
// Thread c < D handles channel c; threads past D load channel D-1 and only
// help with the seal copy.
struct TokenIn {
  uint32_t kv, vv;  // element bits (K/V storage kind), at bit sh of the word
  float ksc;        // fp8: the K element's group scale
  int sh;
};
struct TokenBlock {
  int page;
  uint32_t old_mn, old_mx;  // bits of the block's stored summary of channel c (s > 0)
};

// FIXED: every path issues the same loads, so a caller's wait counts for its
// own loads issued before these stay exact: with ok = false they read the
// readable int32 at `spare` instead and their values are never used, and
// every kind issues one scale load (unused but for fp8).  Without FIXED,
// ok must be true and only the loads the kind needs are issued.
template <int KVK, int D, bool FIXED = false>
__device__ __forceinline__ TokenIn load_token_in(const AppendArgs& a, int b, int g, bool ok = true,
                                                 const int32_t* spare = nullptr) {
  using E = typename ElemT<KVK>::T;
  const long long unit = (long long)b * a.Hkv + g;
  const int c = min((int)threadIdx.x, D - 1);
  TokenIn in;
  in.ksc = 1.0f;
  in.sh = 0;
  if constexpr (FIXED) {
    const E* kp = ok ? static_cast<const E*>(a.k_new) + unit * D + c : reinterpret_cast<const E*>(spare);
    const E* vp = ok ? static_cast<const E*>(a.v_new) + unit * D + c : reinterpret_cast<const E*>(spare);
    const float* sp = ok && KVK == K_FP8 ? a.k_new_scales + unit * (D / a.qg) + c / a.qg
                                         : reinterpret_cast<const float*>(spare);
    in.kv = *kp;
    in.vv = *vp;
    const float sc = *sp;
    if (KVK == K_FP8) in.ksc = sc;
  } else {
    in.kv = static_cast<const E*>(a.k_new)[unit * D + c];
    in.vv = static_cast<const E*>(a.v_new)[unit * D + c];
    if constexpr (KVK == K_FP8) in.ksc = a.k_new_scales[unit * (D / a.qg) + c / a.qg];
  }
  return in;
}

// load_token_in<K_FP8 or K_F32, D, true> with the kind chosen at run time
// (fp32 summaries serve both) and one load sequence for both kinds: each
// element is read as the aligned 32-bit word that holds it (fp8 K/V buffers
// hold whole words: D is a multiple of 4), so the caller's waits stay exact.
template <int D>
__device__ __forceinline__ TokenIn load_token_in_word(const AppendArgs& a, int b, int g, bool ok, bool fp8,
                                                      const int32_t* spare) {
  static_assert(D % 4 == 0, "whole words of fp8 codes per row");
  const long long unit = (long long)b * a.Hkv + g;
  const int c = min((int)threadIdx.x, D - 1);
  const long long e = unit * D + c;                // element index
  const long long off = fp8 ? (e & ~3ll) : 4 * e;  // byte offset of its word
  const int qg = a.qg > 0 ? a.qg : 1;
  const uint32_t* kp = ok ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(a.k_new) + off)
                          : reinterpret_cast<const uint32_t*>(spare);
  const uint32_t* vp = ok ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(a.v_new) + off)
                          : reinterpret_cast<const uint32_t*>(spare);
  const float* sp = ok && fp8 ? a.k_new_scales + unit * (D / qg) + c / qg : reinterpret_cast<const float*>(spare);
  TokenIn in;
  in.kv = *kp;
  in.vv = *vp;
  const float sc = *sp;
  in.ksc = fp8 ? sc : 1.0f;
  in.sh = fp8 ? 8 * (int)(e & 3) : 0;
  return in;
}

// SCALAR_PAGE: the table entry is read through the scalar cache (it is the
// same for the whole workgroup), so that it does not queue behind the
// caller's vector loads; the table must not be written during the kernel.
// FIXED and ok as for load_token_in (with ok = false, len is not used).
template <int KVK, int D, bool SCALAR_PAGE, bool FIXED = false>
__device__ __forceinline__ TokenBlock load_token_block(const AppendArgs& a, int b, int g, int len, bool ok = true,
                                                       const int32_t* spare = nullptr) {
  using E = typename std::conditional<KVK == K_BF16, uint16_t, uint32_t>::type;  // summary element
  const long long unit = (long long)b * a.Hkv + g;
  const int c = min((int)threadIdx.x, D - 1);
  const int S = ok ? a.S : 1;  // (a caller's unused arguments may hold zeros)
  const int t = ok ? len - 1 : 0, j = t / S, s = t % S;
  TokenBlock blk;
  const int32_t* te = a.block_table + (long long)b * a.MB + j;
  if (FIXED && !ok) te = spare;
  if constexpr (SCALAR_PAGE)
    blk.page = *(const __attribute__((address_space(4))) int32_t*)te;
  else
    blk.page = *te;
  // the block's stored summary (its tokens before t) is read beside the
  // page, as raw bits: converted only where they are used
  const long long row = (unit * a.MB + j) * 2 * D;  // min at [0, D), max at [D, 2D)
  const bool want = ok && s > 0 && !a.skip_summary;
  blk.old_mn = 0u;
  blk.old_mx = 0u;
  if constexpr (FIXED) {
    const E* pmn = want ? static_cast<const E*>(a.summ) + row + c : reinterpret_cast<const E*>(spare);
    const E* pmx = want ? static_cast<const E*>(a.summ) + row + D + c : reinterpret_cast<const E*>(spare);
    blk.old_mn = *pmn;
    blk.old_mx = *pmx;
  } else if (want) {
    const E* ps = static_cast<const E*>(a.summ) + row;
    blk.old_mn = ps[c];
    blk.old_mx = ps[D + c];
  }
  return blk;
}

// Every thread of the NT-thread workgroup calls it (D <= NT), with len in
// [1, MB*S]; all exits are uniform over the workgroup.  COHERENT_SEAL: the
// workgroup may have read the block's tiles before (through its L1, which
// does not see its own later stores), so the seal reads them back from the
// device-coherent level after a device-scope fence.
template <int KVK, int D, int NT, bool COHERENT_SEAL = false>
__device__ __forceinline__ void store_token(const AppendArgs& a, int b, int g, int len, const TokenIn& in,
                                            const TokenBlock& blk) {
  static_assert(D <= NT, "one thread per channel");
  static_assert(!COHERENT_SEAL || KVK != K_FP8, "the coherent seal copies the K/V tiles only");
  using E = typename ElemT<KVK>::T;
  constexpr int EB = elem_bytes<KVK>();
  const int tid = threadIdx.x;
  const long long unit = (long long)b * a.Hkv + g;
  const int groups = KVK == K_FP8 ? D / a.qg : 0;
  const int c = tid < D ? tid : D - 1;
  const int S = a.S, T = S < 32 ? S : 32;
  const int t = len - 1, j = t / S, s = t % S;
  const int page = blk.page;
  if (page < 0 || page >= a.P) {
    if (tid == 0) raise_flag(a.err, 0x2u);
    return;
  }
  uint32_t kw = in.kv, vw = in.vv;
  // (an empty asm statement: the element extraction stays here, so a caller
  // that loaded the token early does not wait for those loads early)
  asm volatile("" : "+v"(kw), "+v"(vw));
  const E kv = (E)(kw >> in.sh), vv = (E)(vw >> in.sh);
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
      x = f[0] * in.ksc;
    }
    uint32_t omn = blk.old_mn, omx = blk.old_mx;
    // (an empty asm statement: the conversions below stay here, so a caller
    // that loaded the block early does not wait for those loads early)
    asm volatile("" : "+v"(omn), "+v"(omx));
    const float old_mn = KVK == K_BF16 ? bf16_lo(omn) : __uint_as_float(omn);
    const float old_mx = KVK == K_BF16 ? bf16_lo(omx) : __uint_as_float(omx);
    const float mn = s > 0 ? fminf(old_mn, x) : x;
    const float mx = s > 0 ? fmaxf(old_mx, x) : x;
    const long long row = (unit * a.MB + j) * 2 * D;
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
  if constexpr (COHERENT_SEAL) {
    __threadfence();
    for (int i = tid; i < nvec; i += NT) {
      u32x4 x, y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = __hip_atomic_load(reinterpret_cast<const uint32_t*>(sk + i) + e, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        y[e] = __hip_atomic_load(reinterpret_cast<const uint32_t*>(sv + i) + e, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
      dk[i] = x;
      dv[i] = y;
    }
  } else {
    for (int i = tid; i < nvec; i += NT) {
      const u32x4 x = sk[i];
      const u32x4 y = sv[i];
      dk[i] = x;
      dv[i] = y;
    }
  }
  if constexpr (KVK == K_FP8) {
    const long long ns = (long long)S * groups;
    for (int i = tid; i < ns; i += NT) {
      a.host_ks[host_tile * ns + i] = a.k_scales[tile * ns + i];
      a.host_vs[host_tile * ns + i] = a.v_scales[tile * ns + i];
    }
  }
}

// All three phases in a row.  Every thread of the NT-thread workgroup calls
// it (D <= NT); all exits are uniform over the workgroup.
template <int KVK, int D, int NT>
__device__ __forceinline__ void append_token_unit(const AppendArgs& a, int b, int g) {
  // loads that need no length go out with the length itself
  const int len = a.seq_lens[b];
  const TokenIn in = load_token_in<KVK, D>(a, b, g);
  if (len < 0 || len > a.MB * a.S) {
    if (threadIdx.x == 0 && g == 0) raise_flag(a.err, 0x1u);
    return;
  }
  if (len == 0) return;
  const TokenBlock blk = load_token_block<KVK, D, false>(a, b, g, len);
  store_token<KVK, D, NT>(a, b, g, len, in, blk);
}

}  // namespace kvs
