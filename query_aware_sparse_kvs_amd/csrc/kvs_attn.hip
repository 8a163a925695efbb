// kvs_attn.hip -- attention over the selected blocks only (page "KV 稀疏化",
// §5 "Quest", last step), tiled with a running max and normaliser per tile
// that are merged across tiles and splits ("分块稀疏注意力与KV Cache量化…",
// §2.2), fp8 K/V dequantised inside the read (same page, §1.3).
//
// Work split: a (sequence, KV head) unit's k selected blocks are cut into
// `nsplit` runs of `bps` entries; one 256-thread workgroup (4 wavefronts)
// handles one run, each wavefront one block at a time.  For a block:
//   scores   lane = token (64/S lanes share a token and split its channels);
//            the group's G query rows sit in LDS and are read as broadcasts;
//   softmax  per head, wavefront max/sum by shuffles, base-2 exponentials
//            (the query is pre-scaled by sm_scale*log2 e);
//   values   lane = channel pair; the tile's probabilities go through LDS.
// The four wavefronts' (m, l, acc) are merged in LDS and written as a
// split partial; combine_kernel merges the splits of a query head:
//   m* = max m_i, l* = sum l_i 2^(m_i-m*), o = sum acc_i 2^(m_i-m*) / l*.
// Roofline: HBM-bound gather of 2*S*D*elem bytes per selected block.
#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kGMax = 16;

template <int QK, int KVK, int D, int S>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  constexpr int LPT = kWave / S;   // lanes per token in the score phase
  constexpr int CPL = D / LPT;     // channels per lane in the score phase
  constexpr int VEC = Vec16<KVK>::N;
  static_assert(CPL % VEC == 0, "channel split must be whole 16-byte vectors");
  constexpr int VPL = D / kWave;   // channels per lane in the value phase
  constexpr int EB = elem_bytes<KVK>();

  extern __shared__ float smem[];
  const int G = a.G;
  float* qs = smem;                      // [G][D]
  float* ps = qs + G * D;                // [4][G][S]
  float* mg_m = ps + 4 * G * S;          // [4][G]
  float* mg_l = mg_m + 4 * G;            // [4][G]
  float* mg_acc = mg_l + 4 * G;          // [3][G][D] (wavefronts 1..3)

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, c = i % D;
    const long long qi = ((long long)b * a.Hq + (long long)g * G + h) * D + c;
    float v;
    if constexpr (QK == K_F32)
      v = static_cast<const float*>(a.q)[qi];
    else
      v = __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.q)[qi] << 16);
    qs[i] = v * a.q_scale;
  }
  __syncthreads();

  int len = a.seq_lens[b];
  const int cap = a.MB * S;
  if (len < 0 || len > cap) {
    if (tid == 0 && split == 0 && g == 0) raise_flag(a.err, 0x1u);
    len = len < 0 ? 0 : cap;
  }
  const int nb = (len + S - 1) / S;

  float m_run[kGMax], l_run[kGMax], acc[kGMax][VPL];
#pragma unroll
  for (int h = 0; h < kGMax; ++h) {
    m_run[h] = -__builtin_inff();
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) acc[h][e] = 0.0f;
  }

  const int32_t* srow = a.sel + ((long long)b * a.Hkv + g) * a.k;
  const int i0 = split * a.bps;
  const int i1 = min(i0 + a.bps, a.k);
  const int t = lane % S, part = lane / S;
  float* pw = ps + wave * G * S;
  const char* kb = static_cast<const char*>(a.k_pool);
  const char* vb = static_cast<const char*>(a.v_pool);
  const int groups = KVK == K_FP8 ? D / a.qg : 1;

  for (int i = i0 + wave; i < i1; i += 4) {
    const int j = srow[i];
    if (j < 0) {
      if (j != -1 && lane == 0) raise_flag(a.err, 0x4u);
      continue;
    }
    if (j >= nb || (i > 0 && (srow[i - 1] >= j || srow[i - 1] < 0))) {
      if (lane == 0) raise_flag(a.err, 0x4u);
      if (j >= nb) continue;
    }
    const int entry = a.hot ? a.table[((long long)b * a.Hkv + g) * a.MB + j]
                            : a.table[(long long)b * a.MB + j];
    if (entry < 0 || entry >= a.P) {
      if (lane == 0) raise_flag(a.err, 0x2u);
      continue;
    }
    // first token row of the tile, in elements / D
    const long long row0 = a.hot ? (long long)entry * S : ((long long)entry * a.Hkv + g) * S;
    const int ntok = min(S, len - j * S);

    // ---- scores ----
    float dot[kGMax];
#pragma unroll
    for (int h = 0; h < kGMax; ++h) dot[h] = 0.0f;
    if (t < ntok) {
      const long long r = row0 + t;
#pragma unroll
      for (int cc = 0; cc < CPL; cc += VEC) {
        const int c = part * CPL + cc;
        float kv[VEC];
        Vec16<KVK>::load(kb + (r * D + c) * EB, kv);
        if constexpr (KVK == K_FP8) {
          const float sc = a.k_scales[r * groups + c / a.qg];
#pragma unroll
          for (int e = 0; e < VEC; ++e) kv[e] *= sc;
        }
#pragma unroll
        for (int h = 0; h < kGMax; ++h) {
          if (h < G) {
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
              const float4 qv = *reinterpret_cast<const float4*>(qs + h * D + c + e);
              dot[h] += qv.x * kv[e] + qv.y * kv[e + 1] + qv.z * kv[e + 2] + qv.w * kv[e + 3];
            }
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kGMax; ++h) {
      if (h < G) {
#pragma unroll
        for (int off = S; off < kWave; off <<= 1) dot[h] += __shfl_xor(dot[h], off);
      }
    }
    // ---- online softmax (base 2) ----
#pragma unroll
    for (int h = 0; h < kGMax; ++h) {
      if (h < G) {
        const float s = t < ntok ? dot[h] : -__builtin_inff();
        const float mt = wave_max(s);
        const float mnew = fmaxf(m_run[h], mt);
        const float alpha = exp2f(m_run[h] - mnew);
        const float p = exp2f(s - mnew);
        const float psum = wave_sum(part == 0 ? p : 0.0f);
        l_run[h] = l_run[h] * alpha + psum;
        m_run[h] = mnew;
#pragma unroll
        for (int e = 0; e < VPL; ++e) acc[h][e] *= alpha;
        if (part == 0) pw[h * S + t] = p;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- values ----
    const int c0 = lane * VPL;
    for (int tt = 0; tt < ntok; ++tt) {
      float v[VPL];
      const long long r = row0 + tt;
      if constexpr (KVK == K_F32) {
        if constexpr (VPL == 2) {
          const float2 w = *reinterpret_cast<const float2*>(vb + (r * D + c0) * 4);
          v[0] = w.x;
          v[1] = w.y;
        } else {
          v[0] = *reinterpret_cast<const float*>(vb + (r * D + c0) * 4);
        }
      } else if constexpr (KVK == K_BF16) {
        if constexpr (VPL == 2) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(vb + (r * D + c0) * 2);
          v[0] = bf16_lo(w);
          v[1] = bf16_hi(w);
        } else {
          v[0] = __uint_as_float((uint32_t) * reinterpret_cast<const uint16_t*>(vb + (r * D + c0) * 2) << 16);
        }
      } else {
        const float sc = a.v_scales[r * groups + c0 / a.qg];
        if constexpr (VPL == 2) {
          const uint32_t w = *reinterpret_cast<const uint16_t*>(vb + (r * D + c0));
          typedef __attribute__((ext_vector_type(2))) float f2;
          const f2 f = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
          v[0] = f.x * sc;
          v[1] = f.y * sc;
        } else {
          const uint32_t w = *reinterpret_cast<const uint8_t*>(vb + (r * D + c0));
          typedef __attribute__((ext_vector_type(2))) float f2;
          const f2 f = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
          v[0] = f.x * sc;
        }
      }
#pragma unroll
      for (int h = 0; h < kGMax; ++h) {
        if (h < G) {
          const float p = pw[h * S + tt];
#pragma unroll
          for (int e = 0; e < VPL; ++e) acc[h][e] += p * v[e];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the four wavefronts ----
  if (lane == 0) {
    for (int h = 0; h < G; ++h) {
      mg_m[wave * G + h] = m_run[h];
      mg_l[wave * G + h] = l_run[h];
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int h = 0; h < kGMax; ++h)
      if (h < G)
#pragma unroll
        for (int e = 0; e < VPL; ++e) mg_acc[((wave - 1) * G + h) * D + lane * VPL + e] = acc[h][e];
  }
  __syncthreads();
  if (wave != 0) return;
  const long long pbase = ((long long)b * a.Hq + (long long)g * G) * a.nsplit + split;
#pragma unroll
  for (int h = 0; h < kGMax; ++h) {
    if (h >= G) continue;
    float M = mg_m[h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, mg_m[w * G + h]);
    float sc[4];
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mg_m[w * G + h];
      sc[w] = mw == -__builtin_inff() ? 0.0f : exp2f(mw - M);
      L += mg_l[w * G + h] * sc[w];
    }
    const long long pi = pbase + (long long)h * a.nsplit;
    if (lane == 0) {
      a.part_m[pi] = M;
      a.part_l[pi] = L;
    }
#pragma unroll
    for (int e = 0; e < VPL; ++e) {
      float o = acc[h][e] * sc[0];
#pragma unroll
      for (int w = 1; w < 4; ++w) o += mg_acc[((w - 1) * G + h) * D + lane * VPL + e] * sc[w];
      a.part_acc[pi * D + lane * VPL + e] = o;
    }
  }
}

// one workgroup per (sequence, query head); thread c owns output channel c
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  if (c >= a.D) return;
  const long long pbase = ((long long)b * a.Hq + h) * a.nsplit;
  float M = -__builtin_inff();
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_m[pbase + s]);
  float o = 0.0f;
  if (M != -__builtin_inff()) {
    float L = 0.0f, acc = 0.0f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float ms = a.part_m[pbase + s];
      const float w = ms == -__builtin_inff() ? 0.0f : exp2f(ms - M);
      L += a.part_l[pbase + s] * w;
      acc += a.part_acc[(pbase + s) * a.D + c] * w;
    }
    o = acc / L;
  }
  a.out[((long long)b * a.Hq + h) * a.D + c] = o;
}

template <int QK, int KVK, int D>
hipError_t launch_s(const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)a.B);
  const size_t lds = sizeof(float) * ((size_t)a.G * D + 4 * (size_t)a.G * a.S + 8 * (size_t)a.G +
                                      3 * (size_t)a.G * D);
  switch (a.S) {
    case 16: hipLaunchKernelGGL((attn_split_kernel<QK, KVK, D, 16>), grid, dim3(256), lds, st, a); break;
    case 32: hipLaunchKernelGGL((attn_split_kernel<QK, KVK, D, 32>), grid, dim3(256), lds, st, a); break;
    default: hipLaunchKernelGGL((attn_split_kernel<QK, KVK, D, 64>), grid, dim3(256), lds, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)a.Hq, (unsigned)a.B), dim3(128), 0, st, a);
  return hipGetLastError();
}

template <int QK, int KVK>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  return a.D == 64 ? launch_s<QK, KVK, 64>(a, st) : launch_s<QK, KVK, 128>(a, st);
}

}  // namespace

int attn_num_splits(int units, int k) {
  // enough workgroups to cover the 256 compute units several times over,
  // but at least one selected block per wavefront of a split
  const int by_k = (k + 3) / 4;
  int want = (2048 + units - 1) / (units > 0 ? units : 1);
  if (want < 1) want = 1;
  int n = by_k < want ? by_k : want;
  return n < 1 ? 1 : n;
}

hipError_t launch_attn(const AttnArgs& a, int q_kind, int kv_kind, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (q_kind == K_F32 && kv_kind == K_F32) return launch_d<K_F32, K_F32>(a, st);
  if (q_kind == K_BF16 && kv_kind == K_BF16) return launch_d<K_BF16, K_BF16>(a, st);
  return launch_d<K_BF16, K_FP8>(a, st);
}

}  // namespace kvs
