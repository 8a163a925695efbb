// kvs_internal.h -- device helpers and launcher declarations shared by the
// libkvs translation units.  Not part of the public ABI (include/kvs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

// element kinds of q / K / V / summaries
enum Kind : int { K_F32 = 0, K_BF16 = 1, K_FP8 = 2, K_MEAN = 3 /* fp32 mean summaries */ };

constexpr int kWave = 64;

// 16 bytes as a native vector (HIP's uint4 is a struct; copying it whole
// keeps staging arrays out of registers)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// a float that holds a bf16 value exactly -> its 16-bit pattern
__device__ __forceinline__ uint32_t bf16_bits_exact(float f) { return __float_as_uint(f) >> 16; }

// Two OCP E4M3FN codes (bytes 0,1 or 2,3 of w) -> two floats, by the gfx950
// conversion instruction.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* out) {
  typedef __attribute__((ext_vector_type(2))) float f2;
  f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  out[0] = lo.x;
  out[1] = lo.y;
  out[2] = hi.x;
  out[3] = hi.y;
}

// Loads the 16 bytes at p (16-byte aligned) and converts them to floats:
// 4 fp32, 8 bf16 or 16 fp8 elements.
template <int KIND>
struct Vec16 {
  static constexpr int N = KIND == K_F32 ? 4 : (KIND == K_BF16 ? 8 : 16);
  __device__ __forceinline__ static void load(const void* p, float* out) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    if constexpr (KIND == K_F32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(ws[i]);
    } else if constexpr (KIND == K_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = bf16_lo(ws[i]);
        out[2 * i + 1] = bf16_hi(ws[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) fp8x4_to_f32(ws[i], out + 4 * i);
    }
  }
};

template <int KIND>
constexpr int elem_bytes() {
  return KIND == K_F32 ? 4 : (KIND == K_BF16 ? 2 : 1);
}

// ---------------------------------------------------------------------------
// wavefront reductions (64 lanes)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Block-wide exclusive prefix sum for 256-thread blocks.  `tmp` must hold 4
// ints of LDS.  Returns the exclusive prefix of v; *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int t = tmp[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Sets bits in the library's device error word.
__device__ __forceinline__ void raise_flag(unsigned int* word, unsigned int bits) {
  if (word) atomicOr(word, bits);
}

// ---------------------------------------------------------------------------
// launcher argument blocks (plain data, passed by value to kernels)
// ---------------------------------------------------------------------------

struct SummArgs {
  const void* k_pool;
  const float* k_scales;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* first_block;
  void* out;
  unsigned int* err;
  int32_t B, Hkv, D, S, MB, P, qg, num_rebuild;
  int32_t newest;  // 1: rebuild block nb(b)-1 of every sequence (first_block unused)
  int32_t mean;    // 1: the fp32 mean table [B][Hkv][MB][D] instead of min/max
};

// One decode token per sequence written into its page, its block's summary
// updated, and a block that has just filled copied to the host tier.
struct AppendArgs {
  const void* k_new;            // [B][Hkv][D] K/V storage kind
  const void* v_new;
  const float* k_new_scales;    // fp8: [B][Hkv][D/qg]
  const float* v_new_scales;
  const int32_t* block_table;   // [B][MB]
  const int32_t* seq_lens;      // [B], the new token included
  void* k_pool;                 // [P][Hkv][S][D]
  void* v_pool;                 // [P][Hkv][S/T][D][T]
  float* k_scales;              // fp8: [P][Hkv][S][D/qg]
  float* v_scales;
  void* summ;                   // [B][Hkv][MB][2][D], bf16 for bf16 K else fp32
  void* host_k;                 // device aliases of the pinned host tier, or null
  void* host_v;
  float* host_ks;
  float* host_vs;
  unsigned int* err;
  int32_t B, Hkv, D, S, MB, P, qg;
  int32_t skip_summary;  // 1: K/V (and the seal) only; the caller rebuilds the summary
};

struct BoundArgs {
  const void* q;
  const void* summ;
  const int32_t* seq_lens;
  double* W;           // workspace [B][Hkv][MB]
  double* bounds_out;  // optional copy
  unsigned int* err;
  int32_t B, Hq, Hkv, D, S, MB;
  int32_t append;      // 1: one more workgroup per (b, g) rebuilds the newest block's
                       // summary (app); 2: the first workgroup of each (b, g) also
                       // appends the decode token (tok)
  int32_t app_kv;      // K storage kind of that work (Kind; bf16 with bf16 summaries)
  SummArgs app;
  AppendArgs tok;
  int32_t ema;         // 1: W is smoothed with ema_state before it is stored
  double ema_alpha;    // weight of this step's score
  double ema_beta;     // 1 - ema_alpha (fp64)
  double* ema_state;   // [B][Hkv][MB] in/out, NaN = no history
  int32_t accumulate;  // 1: W[j] = W[j] + this launch's score (cross-layer
                       // fusion), for j < nb; W holds the earlier layers' sum
};

struct TopkArgs {
  const double* W;
  const int32_t* seq_lens;
  int32_t* sel;
  int32_t B, Hkv, S, MB, k;
  int32_t recent;  // newest blocks always kept (>= 1)
};

struct SelMfmaArgs {
  const void* q;
  const void* summ;
  const int32_t* seq_lens;
  float* w32;   // workspace [B][Hkv][MB]: fp32 scores
  float* amag;  // workspace [B][Hkv][MB]: their error magnitudes
  int32_t* sel;
  unsigned int* err;
  int32_t B, Hq, Hkv, G, D, S, MB, k;
  int32_t recent;  // as in TopkArgs
  int32_t append;  // 1 / 2 as in BoundArgs, both done by one more workgroup per (b, g)
  SummArgs app;
  AppendArgs tok;
};

struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const float* k_scales;
  const float* v_scales;
  const int32_t* table;
  const int32_t* seq_lens;
  const int32_t* sel;
  float* part_m;    // [B][Hq][nsplit]
  float* part_l;    // [B][Hq][nsplit]
  float* part_acc;  // [B][Hq][nsplit][D]
  float* out;       // [B][Hq][D]
  unsigned int* err;
  float q_scale;    // sm_scale * log2(e): scores are kept in base 2
  int32_t B, Hq, Hkv, G, D, S, MB, P, qg, k, nsplit, bps, hot;
  // self-selecting mode (W non-null): every workgroup selects its unit's
  // blocks from the scores W [B][Hkv][MB] (recent = newest blocks always
  // kept), and the first split's workgroup writes the selection to sel_out
  const double* W;
  int32_t* sel_out;
  int32_t recent;
};

struct HotArgs {
  const int32_t* sel;
  int32_t* pt;
  int32_t* owner;
  int64_t* stamp;
  int32_t* miss_list;
  int32_t* miss_count;
  const void* host_k;
  const void* host_v;
  const float* host_ks;
  const float* host_vs;
  void* hot_k;
  void* hot_v;
  float* hot_ks;
  float* hot_vs;
  unsigned int* err;
  int64_t step;
  int32_t B, Hkv, D, S, MB, k, ns, n2, qg, elem_bytes;
  // the paged cache each unit's newest block is copied from (live_k null:
  // every block comes from the host tier)
  const void* live_k;
  const void* live_v;
  const float* live_ks;
  const float* live_vs;
  const int32_t* live_table;  // [B][MB]
  const int32_t* live_lens;   // [B]
  int32_t P;                  // pages of that cache
};

// launchers (return the launch status); kinds/shapes are validated by the
// caller
hipError_t launch_summaries(const SummArgs& a, int kv_kind, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, int kv_kind, hipStream_t s);
hipError_t launch_bounds(const BoundArgs& a, int q_kind, int summ_kind, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
bool select_mfma_supported(int q_kind, int summ_kind, int D, int MB, int G);
hipError_t launch_select_mfma(const SelMfmaArgs& a, int summ_kind, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int q_kind, int kv_kind, hipStream_t s);
// whether launch_attn can run this shape in self-selecting mode
bool attn_self_select_supported(int q_kind, int kv_kind, int S, int MB, int k);
// attention over a given selection with the decode token appended in the
// same launch (bf16 K/V, blocks of 32 or 64 tokens, paged table)
bool attn_tok_supported(int q_kind, int kv_kind, int S, int D, int hot);
hipError_t launch_attn_tok(const AttnArgs& a, const AppendArgs& t, int q_kind, int kv_kind, hipStream_t s);
// hot-buffer phases: the page-table step (hits, miss list, LRU victims) and
// the copy of the listed misses from the host tier
constexpr int kHotLookup = 1, kHotCopy = 2;
hipError_t launch_hot(const HotArgs& a, int phases, hipStream_t s);

// attention split heuristic shared by the launcher and the workspace query
int attn_num_splits(int units, int k);

}  // namespace kvs
