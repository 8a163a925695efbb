// kvs_api.hip -- the extern "C" entry points declared in include/kvs.h:
// host-side argument validation, dtype/shape dispatch, workspace sizing,
// status strings and the device error word.  No allocation happens here;
// every buffer belongs to the caller.
#include <mutex>
#include <string>

#include "kvs.h"
#include "kvs_internal.h"

// OR of KVS_DEVERR_* bits raised by kernels on this device.
__device__ unsigned int kvs_device_error_word = 0u;

// The allocation-free attention entry point keeps its split partials in
// this file-scope array, one copy per GPU (the code object is loaded on
// every device the library runs on) that lives until the process ends.
// Several splits per (sequence, KV head) only happen while B*Hkv < 256
// compute units, so B*Hq*nsplit < 16*512 rows of (2 + D) floats: at most
// 4.25 MiB for D = 128.  Host code uses the per-device address from
// hipGetSymbolAddress, never the name.
static __device__ __align__(256) unsigned char scratch[KVS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

kvs_status fail(kvs_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

kvs_status ok() {
  g_last_error.clear();
  return KVS_OK;
}

// device address of kvs_device_error_word, looked up once per device
constexpr int kMaxDevices = 64;
unsigned int* g_err_word[kMaxDevices] = {};
std::mutex g_err_mu;

kvs_status error_word(unsigned int** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVS_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_err_mu);
  if (!g_err_word[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(kvs_device_error_word));
    if (e != hipSuccess || !p)
      return fail(KVS_ERR_HIP, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_err_word[dev] = static_cast<unsigned int*>(p);
  }
  *out = g_err_word[dev];
  return KVS_OK;
}

kvs_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int kind_of(int32_t dt) {
  switch (dt) {
    case KVS_F32: return kvs::K_F32;
    case KVS_BF16: return kvs::K_BF16;
    default: return kvs::K_FP8;
  }
}

size_t elem_size(int32_t dt) { return dt == KVS_F32 ? 4 : (dt == KVS_BF16 ? 2 : 1); }

// Checks the layout fields every call needs.  `need_q` adds the query-side
// checks (heads, q dtype pairing).
kvs_status check_layout(const kvs_layout* L, bool need_q) {
  if (!L) return fail(KVS_ERR_INVALID_ARG, "layout is NULL");
  if (L->num_seqs < 0) return fail(KVS_ERR_INVALID_ARG, "num_seqs < 0");
  if (L->num_kv_heads < 1) return fail(KVS_ERR_INVALID_ARG, "num_kv_heads < 1");
  if (L->max_blocks < 1 || L->max_blocks > 8192)
    return fail(L->max_blocks < 1 ? KVS_ERR_INVALID_ARG : KVS_ERR_UNSUPPORTED,
                "max_blocks must be in [1, 8192]");
  if (L->num_pages < 1) return fail(KVS_ERR_INVALID_ARG, "num_pages < 1");
  if (L->head_dim != 64 && L->head_dim != 128)
    return fail(L->head_dim <= 0 ? KVS_ERR_INVALID_ARG : KVS_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (L->block_size != 16 && L->block_size != 32 && L->block_size != 64)
    return fail(L->block_size <= 0 ? KVS_ERR_INVALID_ARG : KVS_ERR_UNSUPPORTED,
                "block_size must be 16, 32 or 64");
  if (L->kv_dtype < KVS_F32 || L->kv_dtype > KVS_FP8_E4M3)
    return fail(KVS_ERR_INVALID_ARG, "unknown kv_dtype");
  if (L->kv_dtype == KVS_FP8_E4M3) {
    const int qg = L->quant_group;
    if (qg != 16 && qg != 32 && qg != 64 && qg != 128)
      return fail(KVS_ERR_UNSUPPORTED, "fp8 quant_group must be 16, 32, 64 or 128");
    if (L->head_dim % qg != 0) return fail(KVS_ERR_INVALID_ARG, "quant_group must divide head_dim");
  } else if (L->quant_group != 0) {
    return fail(KVS_ERR_INVALID_ARG, "quant_group must be 0 unless kv_dtype is fp8");
  }
  if ((long long)L->max_blocks * L->block_size > 0x7FFFFFFFll)
    return fail(KVS_ERR_INVALID_ARG, "max_blocks * block_size overflows int32");
  if (need_q) {
    if (L->num_q_heads < 1 || L->num_q_heads % L->num_kv_heads != 0)
      return fail(KVS_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
    const int G = L->num_q_heads / L->num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
      return fail(KVS_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4, 8 or 16");
    if (L->q_dtype != KVS_F32 && L->q_dtype != KVS_BF16) return fail(KVS_ERR_UNSUPPORTED, "q_dtype must be fp32 or bf16");
    const bool pair_ok = (L->q_dtype == KVS_F32 && L->kv_dtype == KVS_F32) ||
                         (L->q_dtype == KVS_BF16 && L->kv_dtype == KVS_BF16) ||
                         (L->q_dtype == KVS_BF16 && L->kv_dtype == KVS_FP8_E4M3);
    if (!pair_ok) return fail(KVS_ERR_UNSUPPORTED, "unsupported (q_dtype, kv_dtype) pair");
  }
  if ((long long)L->num_seqs * L->num_kv_heads > 0x7FFFFFFFll)
    return fail(KVS_ERR_INVALID_ARG, "num_seqs * num_kv_heads overflows int32");
  return KVS_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// (sequences x KV heads x max_blocks) from which kvs_select_topk scores on the
// matrix cores when no bounds are requested
constexpr long long kSelectMfmaMinBlocks = 65536;
// the same for fp32 summaries (fp8 K, the summaries split into two bf16
// parts on the matrix cores).  Measured on MI355X (4 KV heads, 2048 blocks
// per row, k = 64): 32 768 blocks 24.8 us against 17.2 exact, 131 072 41.6
// against 38.3, 262 144 61.2 against 63.0.
constexpr long long kSelectMfmaMinBlocksF32 = 262144;

size_t select_ws(const kvs_layout* L) {
  return round_up(sizeof(double) * (size_t)L->num_seqs * L->num_kv_heads * L->max_blocks, 256);
}

int attn_splits(const kvs_layout* L, int32_t k) {
  return kvs::attn_num_splits(L->num_seqs * L->num_kv_heads, k);
}

// attention workspace: [split m, l][split acc].  With one split the kernels
// write the output rows directly and never touch it (256 bytes are still
// asked for, so that a workspace pointer always exists).
size_t attn_ws(const kvs_layout* L, int32_t k) {
  const int nsplit = attn_splits(L, k);
  if (nsplit == 1) return 256;
  const size_t units = (size_t)L->num_seqs * L->num_q_heads * nsplit;
  return round_up(sizeof(float) * units * 2, 256) + round_up(sizeof(float) * units * L->head_dim, 256);
}

constexpr size_t kNoAllocScratchBytes = KVS_NOALLOC_SCRATCH_BYTES;

// device address of `scratch`, looked up once per device; the array's name
// is only a host-side stand-in and is never passed to a kernel
void* g_scratch[kMaxDevices] = {};

kvs_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVS_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_err_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVS_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KVS_OK;
}

}  // namespace

extern "C" {

int32_t kvs_abi_version(void) { return KVS_ABI_VERSION; }

const char* kvs_status_string(kvs_status st) {
  switch (st) {
    case KVS_OK: return "KVS_OK";
    case KVS_ERR_INVALID_ARG: return "KVS_ERR_INVALID_ARG: invalid argument";
    case KVS_ERR_UNSUPPORTED: return "KVS_ERR_UNSUPPORTED: shape or dtype not supported";
    case KVS_ERR_CAPACITY: return "KVS_ERR_CAPACITY: more blocks than hot slots";
    case KVS_ERR_HIP: return "KVS_ERR_HIP: HIP runtime error";
  }
  return "unknown kvs_status";
}

const char* kvs_last_error(void) { return g_last_error.c_str(); }

size_t kvs_select_workspace_size(const kvs_layout* L, int32_t k) {
  if (check_layout(L, true) != KVS_OK || k < 2 || k > L->max_blocks) return 0;
  return select_ws(L);
}

size_t kvs_attn_workspace_size(const kvs_layout* L, int32_t k) {
  if (check_layout(L, true) != KVS_OK || k < 1 || k > L->max_blocks) return 0;
  return attn_ws(L, k);
}

int32_t kvs_attn_num_splits(const kvs_layout* L, int32_t k) {
  if (check_layout(L, true) != KVS_OK || k < 1 || k > L->max_blocks) return 0;
  return attn_splits(L, k);
}

kvs_status kvs_device_errors(uint32_t* flags, int32_t clear, void* stream) {
  if (!flags) return fail(KVS_ERR_INVALID_ARG, "flags is NULL");
  unsigned int* w = nullptr;
  kvs_status st = error_word(&w);
  if (st != KVS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned int host = 0;
  hipError_t e = hipMemcpyAsync(&host, w, sizeof host, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "reading the device error word");
  *flags = host;
  if (clear) {
    const unsigned int zero = 0;
    e = hipMemcpyAsync(w, &zero, sizeof zero, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "clearing the device error word");
  }
  return ok();
}

kvs_status kvs_build_summaries(const kvs_layout* L, const void* k_pool, const float* k_scales,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* first_block, int32_t num_rebuild, void* summaries,
                               void* stream) {
  return kvs_build_summaries_ex(L, KVS_SUMM_MINMAX, k_pool, k_scales, block_table, seq_lens, first_block,
                                num_rebuild, summaries, stream);
}

kvs_status kvs_build_summaries_ex(const kvs_layout* L, int32_t summary_kind, const void* k_pool,
                                  const float* k_scales, const int32_t* block_table, const int32_t* seq_lens,
                                  const int32_t* first_block, int32_t num_rebuild, void* summaries,
                                  void* stream) {
  if (summary_kind != KVS_SUMM_MINMAX && summary_kind != KVS_SUMM_MEAN)
    return fail(KVS_ERR_INVALID_ARG, "unknown summary_kind");
  kvs_status st = check_layout(L, false);
  if (st != KVS_OK) return st;
  if (!k_pool || !block_table || !seq_lens || !summaries)
    return fail(KVS_ERR_INVALID_ARG, "k_pool, block_table, seq_lens and summaries must be non-NULL");
  if (L->kv_dtype == KVS_FP8_E4M3 && !k_scales) return fail(KVS_ERR_INVALID_ARG, "fp8 K needs k_scales");
  if (num_rebuild < 0 || num_rebuild > L->max_blocks)
    return fail(KVS_ERR_INVALID_ARG, "num_rebuild must be in [0, max_blocks]");
  if (!aligned(k_pool, 16) || !aligned(summaries, 16))
    return fail(KVS_ERR_INVALID_ARG, "k_pool and summaries must be 16-byte aligned");
  unsigned int* err = nullptr;
  if ((st = error_word(&err)) != KVS_OK) return st;
  kvs::SummArgs a{};
  a.k_pool = k_pool;
  a.k_scales = k_scales;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.first_block = first_block;
  a.out = summaries;
  a.err = err;
  a.B = L->num_seqs;
  a.Hkv = L->num_kv_heads;
  a.D = L->head_dim;
  a.S = L->block_size;
  a.MB = L->max_blocks;
  a.P = L->num_pages;
  a.qg = L->quant_group;
  a.num_rebuild = num_rebuild;
  a.mean = summary_kind == KVS_SUMM_MEAN ? 1 : 0;
  return hip_status(kvs::launch_summaries(a, kind_of(L->kv_dtype), static_cast<hipStream_t>(stream)),
                    "summaries launch");
}

}  // extern "C"

namespace {

// Validates a kvs_append_args block and fills the kernels' argument block
// (the host tier is passed to the kernels through its device aliases).
kvs_status make_append(const kvs_layout* L, const kvs_append_args* ap, const int32_t* seq_lens, void* summaries,
                       kvs::AppendArgs* out) {
  if (!ap || !seq_lens || !summaries) return fail(KVS_ERR_INVALID_ARG, "append, seq_lens and summaries must be non-NULL");
  if (!ap->k_new || !ap->v_new || !ap->block_table || !ap->k_pool || !ap->v_pool)
    return fail(KVS_ERR_INVALID_ARG, "k_new, v_new, block_table, k_pool and v_pool must be non-NULL");
  const bool fp8 = L->kv_dtype == KVS_FP8_E4M3;
  if (fp8 && (!ap->k_new_scales || !ap->v_new_scales || !ap->k_scales || !ap->v_scales))
    return fail(KVS_ERR_INVALID_ARG, "fp8 K/V need new-token and pool scales");
  if ((ap->host_k != nullptr) != (ap->host_v != nullptr))
    return fail(KVS_ERR_INVALID_ARG, "host_k and host_v must both be given or both be NULL");
  if (ap->host_k && fp8 && (!ap->host_k_scales || !ap->host_v_scales))
    return fail(KVS_ERR_INVALID_ARG, "an fp8 host tier needs host scales");
  if (!aligned(ap->k_pool, 16) || !aligned(ap->v_pool, 16) || !aligned(summaries, 16) ||
      (ap->host_k && (!aligned(ap->host_k, 16) || !aligned(ap->host_v, 16))))
    return fail(KVS_ERR_INVALID_ARG, "pools, summaries and host tier must be 16-byte aligned");
  void* dev[4] = {nullptr, nullptr, nullptr, nullptr};
  if (ap->host_k) {
    void* host[4] = {ap->host_k, ap->host_v, ap->host_k_scales, ap->host_v_scales};
    for (int i = 0; i < (fp8 ? 4 : 2); ++i) {
      hipError_t e = hipHostGetDevicePointer(&dev[i], host[i], 0);
      if (e != hipSuccess || !dev[i]) {
        (void)hipGetLastError();
        return fail(KVS_ERR_INVALID_ARG, "the host tier must be pinned host memory (hipHostMalloc)");
      }
    }
  }
  kvs::AppendArgs a{};
  a.k_new = ap->k_new;
  a.v_new = ap->v_new;
  a.k_new_scales = ap->k_new_scales;
  a.v_new_scales = ap->v_new_scales;
  a.block_table = ap->block_table;
  a.seq_lens = seq_lens;
  a.k_pool = ap->k_pool;
  a.v_pool = ap->v_pool;
  a.k_scales = ap->k_scales;
  a.v_scales = ap->v_scales;
  a.summ = summaries;
  a.host_k = dev[0];
  a.host_v = dev[1];
  a.host_ks = static_cast<float*>(dev[2]);
  a.host_vs = static_cast<float*>(dev[3]);
  a.B = L->num_seqs;
  a.Hkv = L->num_kv_heads;
  a.D = L->head_dim;
  a.S = L->block_size;
  a.MB = L->max_blocks;
  a.P = L->num_pages;
  a.qg = fp8 ? L->quant_group : 0;
  *out = a;
  return KVS_OK;
}

// Whether the selection scores on the matrix cores (no bounds requested,
// min/max summaries, no smoothing).
bool uses_matrix_cores(const kvs_layout* L, long long blocks, int summ_kind, int G) {
  const long long min_blocks = summ_kind == kvs::K_F32 ? kSelectMfmaMinBlocksF32 : kSelectMfmaMinBlocks;
  return blocks >= min_blocks &&
         kvs::select_mfma_supported(kind_of(L->q_dtype), summ_kind, L->head_dim, L->max_blocks, G);
}

// Selection options after validation.
struct SelectOpts {
  int recent = 1;
  bool ema = false;
  double alpha = 1.0;
  double* state = nullptr;
  int kind = KVS_SUMM_MINMAX;
  bool accumulate = false;
};

SelectOpts opts_of(const kvs_select_opts* opts) {
  SelectOpts o;
  if (opts) {
    o.recent = opts->recent_blocks;
    o.ema = opts->use_ema != 0;
    o.alpha = opts->ema_alpha;
    o.state = opts->ema_state;
    o.kind = opts->summary_kind;
    o.accumulate = opts->accumulate != 0;
  }
  return o;
}

// kvs_select_topk's checks and launches.  With `app`, each sequence's newest
// block summary is also rebuilt from K; with `tok`, the decode token is
// appended -- either by one more workgroup per (sequence, KV head) inside the
// scoring launch (no bounds returned, no smoothing), else by a launch of its
// own before scoring.
kvs_status select_impl(const kvs_layout* L, const void* q, const void* summaries, const int32_t* seq_lens, int32_t k,
                       int32_t* sel, double* bounds_out, void* workspace, size_t workspace_bytes, void* stream,
                       const kvs::SummArgs* app, const SelectOpts& opt, const kvs_append_args* tok_in,
                       double* scores_out = nullptr) {
  // scores_out: stop after the (exact) scores, written there; no selection
  kvs_status st = check_layout(L, true);
  if (st != KVS_OK) return st;
  if (!q || !summaries || !seq_lens || (!sel && !scores_out))
    return fail(KVS_ERR_INVALID_ARG, "q, summaries, seq_lens and sel must be non-NULL");
  if (!scores_out) {
    if (k < 2 || k > L->max_blocks) return fail(KVS_ERR_INVALID_ARG, "k must be in [2, max_blocks]");
    if (opt.recent < 1 || k < opt.recent + 1)
      return fail(KVS_ERR_INVALID_ARG, "recent_blocks must be >= 1 and k >= recent_blocks + 1");
    if (!workspace || workspace_bytes < select_ws(L))
      return fail(KVS_ERR_INVALID_ARG, "workspace missing or smaller than kvs_select_workspace_size()");
  } else if (!aligned(scores_out, 8)) {
    return fail(KVS_ERR_INVALID_ARG, "scores must be 8-byte aligned");
  }
  if (opt.ema && (!opt.state || !aligned(opt.state, 8) || !(opt.alpha >= 0.0 && opt.alpha <= 1.0)))
    return fail(KVS_ERR_INVALID_ARG, "smoothing needs an 8-byte aligned ema_state and 0 <= ema_alpha <= 1");
  if (opt.kind != KVS_SUMM_MINMAX && opt.kind != KVS_SUMM_MEAN)
    return fail(KVS_ERR_INVALID_ARG, "unknown summary_kind");
  if (opt.accumulate && !scores_out)
    return fail(KVS_ERR_INVALID_ARG, "accumulate applies to kvs_score_blocks only");
  const bool mean = opt.kind == KVS_SUMM_MEAN;
  if (mean && app) return fail(KVS_ERR_UNSUPPORTED, "the newest-block rebuild call keeps min/max summaries");
  if (!aligned(summaries, 16) || (workspace && !aligned(workspace, 16)) || (bounds_out && !aligned(bounds_out, 8)))
    return fail(KVS_ERR_INVALID_ARG, "summaries/workspace must be 16-byte aligned, bounds_out 8-byte");
  kvs::AppendArgs tok{};
  if (tok_in && (st = make_append(L, tok_in, seq_lens, const_cast<void*>(summaries), &tok)) != KVS_OK) return st;
  unsigned int* err = nullptr;
  if ((st = error_word(&err)) != KVS_OK) return st;
  tok.err = err;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int summ_kind = mean ? kvs::K_MEAN : (L->kv_dtype == KVS_BF16 ? kvs::K_BF16 : kvs::K_F32);
  const int G = L->num_q_heads / L->num_kv_heads;
  kvs::SummArgs ap{};
  int fuse = 0;  // the scoring launch's extra-workgroup role (BoundArgs::append)
  if (app) {
    ap = *app;
    ap.err = err;
    fuse = bounds_out ? 0 : 1;
    if (!fuse) {  // bounds must see the new summary: rebuild it first
      hipError_t e = kvs::launch_summaries(ap, kind_of(L->kv_dtype), s);
      if (e != hipSuccess) return hip_status(e, "summaries launch");
    }
  } else if (tok_in && mean) {
    // a mean cannot be updated in place exactly: write the token, then
    // rebuild its block's mean from the pool
    tok.skip_summary = 1;
    hipError_t e = kvs::launch_append(tok, kind_of(L->kv_dtype), s);
    if (e != hipSuccess) return hip_status(e, "append launch");
    kvs::SummArgs ms{};
    ms.k_pool = tok.k_pool;
    ms.k_scales = tok.k_scales;
    ms.block_table = tok.block_table;
    ms.seq_lens = seq_lens;
    ms.out = const_cast<void*>(summaries);
    ms.err = err;
    ms.B = L->num_seqs;
    ms.Hkv = L->num_kv_heads;
    ms.D = L->head_dim;
    ms.S = L->block_size;
    ms.MB = L->max_blocks;
    ms.P = L->num_pages;
    ms.qg = L->quant_group;
    ms.num_rebuild = 1;
    ms.newest = 1;
    ms.mean = 1;
    e = kvs::launch_summaries(ms, kind_of(L->kv_dtype), s);
    if (e != hipSuccess) return hip_status(e, "summaries launch");
  } else if (tok_in) {
    // fused only where the newest block's racing score is never used: it
    // would reach bounds_out, and through smoothing the next steps
    fuse = (bounds_out || opt.ema) ? 0 : 2;
    if (!fuse) {
      hipError_t e = kvs::launch_append(tok, kind_of(L->kv_dtype), s);
      if (e != hipSuccess) return hip_status(e, "append launch");
    }
  }
  // Two implementations with identical selections.  The exact one spends a
  // fixed amount of fp64 arithmetic per (block, head, channel); the
  // matrix-core one streams the summaries at memory speed but pays a longer
  // per-unit selection.  Measured on MI355X the second wins from a few tens
  // of thousands of blocks (8 x 4 x 512: 15.0 vs 16.5 us; 256 x 4 x 512:
  // 108 vs 75 us).
  const long long blocks = (long long)L->num_seqs * L->num_kv_heads * L->max_blocks;
  if (!scores_out && !bounds_out && !opt.ema && !mean && uses_matrix_cores(L, blocks, summ_kind, G)) {
    kvs::SelMfmaArgs ma{};
    ma.q = q;
    ma.summ = summaries;
    ma.seq_lens = seq_lens;
    ma.w32 = static_cast<float*>(workspace);
    ma.amag = ma.w32 + (size_t)L->num_seqs * L->num_kv_heads * L->max_blocks;
    ma.sel = sel;
    ma.err = err;
    ma.B = L->num_seqs;
    ma.Hq = L->num_q_heads;
    ma.Hkv = L->num_kv_heads;
    ma.G = G;
    ma.D = L->head_dim;
    ma.S = L->block_size;
    ma.MB = L->max_blocks;
    ma.k = k;
    ma.recent = opt.recent;
    ma.append = fuse;
    ma.app = ap;
    ma.tok = tok;
    return hip_status(kvs::launch_select_mfma(ma, summ_kind, s), "select launch");
  }
  kvs::BoundArgs ba{};
  ba.q = q;
  ba.summ = summaries;
  ba.seq_lens = seq_lens;
  ba.W = scores_out ? scores_out : static_cast<double*>(workspace);
  ba.bounds_out = bounds_out;
  ba.err = err;
  ba.B = L->num_seqs;
  ba.Hq = L->num_q_heads;
  ba.Hkv = L->num_kv_heads;
  ba.D = L->head_dim;
  ba.S = L->block_size;
  ba.MB = L->max_blocks;
  ba.append = fuse;
  ba.app_kv = kind_of(L->kv_dtype);
  ba.app = ap;
  ba.tok = tok;
  ba.ema = opt.ema ? 1 : 0;
  ba.ema_alpha = opt.alpha;
  ba.ema_beta = 1.0 - opt.alpha;
  ba.ema_state = opt.state;
  ba.accumulate = opt.accumulate ? 1 : 0;
  hipError_t e = kvs::launch_bounds(ba, kind_of(L->q_dtype), summ_kind, s);
  if (e != hipSuccess || scores_out) return hip_status(e, "bounds launch");
  kvs::TopkArgs ta{};
  ta.W = ba.W;
  ta.seq_lens = seq_lens;
  ta.sel = sel;
  ta.B = L->num_seqs;
  ta.Hkv = L->num_kv_heads;
  ta.S = L->block_size;
  ta.MB = L->max_blocks;
  ta.k = k;
  ta.recent = opt.recent;
  return hip_status(kvs::launch_topk(ta, s), "top-k launch");
}

}  // namespace

extern "C" {

int32_t kvs_select_uses_matrix_cores(const kvs_layout* L, int32_t k) {
  if (check_layout(L, true) != KVS_OK || k < 2 || k > L->max_blocks) return 0;
  const int summ_kind = L->kv_dtype == KVS_BF16 ? kvs::K_BF16 : kvs::K_F32;
  const long long blocks = (long long)L->num_seqs * L->num_kv_heads * L->max_blocks;
  return uses_matrix_cores(L, blocks, summ_kind, L->num_q_heads / L->num_kv_heads) ? 1 : 0;
}

kvs_status kvs_select_topk(const kvs_layout* L, const void* q, const void* summaries,
                           const int32_t* seq_lens, int32_t k, int32_t* sel, double* bounds_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl(L, q, summaries, seq_lens, k, sel, bounds_out, workspace, workspace_bytes, stream, nullptr,
                     SelectOpts{}, nullptr);
}

kvs_status kvs_select_topk_ex(const kvs_layout* L, const void* q, void* summaries, const int32_t* seq_lens,
                              int32_t k, const kvs_select_opts* opts, const kvs_append_args* append, int32_t* sel,
                              double* bounds_out, void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl(L, q, summaries, seq_lens, k, sel, bounds_out, workspace, workspace_bytes, stream, nullptr,
                     opts_of(opts), append);
}

kvs_status kvs_append_token(const kvs_layout* L, const kvs_append_args* append, const int32_t* seq_lens,
                            void* summaries, void* stream) {
  kvs_status st = check_layout(L, false);
  if (st != KVS_OK) return st;
  kvs::AppendArgs a{};
  if ((st = make_append(L, append, seq_lens, summaries, &a)) != KVS_OK) return st;
  unsigned int* err = nullptr;
  if ((st = error_word(&err)) != KVS_OK) return st;
  a.err = err;
  return hip_status(kvs::launch_append(a, kind_of(L->kv_dtype), static_cast<hipStream_t>(stream)), "append launch");
}

kvs_status kvs_select_topk_append(const kvs_layout* L, const void* q, const void* k_pool, const float* k_scales,
                                  const int32_t* block_table, const int32_t* seq_lens, void* summaries,
                                  int32_t k, int32_t* sel, double* bounds_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  kvs_status st = check_layout(L, true);
  if (st != KVS_OK) return st;
  if (!k_pool || !block_table) return fail(KVS_ERR_INVALID_ARG, "k_pool and block_table must be non-NULL");
  if (L->kv_dtype == KVS_FP8_E4M3 && !k_scales) return fail(KVS_ERR_INVALID_ARG, "fp8 K needs k_scales");
  if (!aligned(k_pool, 16)) return fail(KVS_ERR_INVALID_ARG, "k_pool must be 16-byte aligned");
  kvs::SummArgs ap{};
  ap.k_pool = k_pool;
  ap.k_scales = k_scales;
  ap.block_table = block_table;
  ap.seq_lens = seq_lens;
  ap.first_block = nullptr;
  ap.out = summaries;
  ap.B = L->num_seqs;
  ap.Hkv = L->num_kv_heads;
  ap.D = L->head_dim;
  ap.S = L->block_size;
  ap.MB = L->max_blocks;
  ap.P = L->num_pages;
  ap.qg = L->quant_group;
  ap.num_rebuild = 1;
  ap.newest = 1;
  return select_impl(L, q, summaries, seq_lens, k, sel, bounds_out, workspace, workspace_bytes, stream, &ap,
                     SelectOpts{}, nullptr);
}

}  // extern "C"

namespace {
kvs_status attn_impl(const kvs_layout* L, int32_t table_kind, const void* q, const void* k_pool, const void* v_pool,
                     const float* k_scales, const float* v_scales, const int32_t* table, const int32_t* seq_lens,
                     const int32_t* sel, int32_t k, float sm_scale, float* out, void* workspace,
                     size_t workspace_bytes, void* stream, const double* scores, int32_t recent,
                     bool noalloc = false, const kvs::AppendArgs* tok = nullptr);
}  // namespace

extern "C" {

kvs_status kvs_sparse_decode_attn(const kvs_layout* L, int32_t table_kind, const void* q,
                                  const void* k_pool, const void* v_pool, const float* k_scales,
                                  const float* v_scales, const int32_t* table, const int32_t* seq_lens,
                                  const int32_t* sel, int32_t k, float sm_scale, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return attn_impl(L, table_kind, q, k_pool, v_pool, k_scales, v_scales, table, seq_lens, sel, k, sm_scale, out,
                   workspace, workspace_bytes, stream, nullptr, 0);
}

kvs_status kvs_append_sparse_decode_attn(const kvs_layout* L, const kvs_append_args* append, void* summaries,
                                         const void* q, const int32_t* seq_lens, const int32_t* sel, int32_t k,
                                         float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  kvs_status st = check_layout(L, true);
  if (st != KVS_OK) return st;
  kvs::AppendArgs t{};
  if ((st = make_append(L, append, seq_lens, summaries, &t)) != KVS_OK) return st;
  return attn_impl(L, KVS_TABLE_PAGED, q, append->k_pool, append->v_pool, append->k_scales, append->v_scales,
                   append->block_table, seq_lens, sel, k, sm_scale, out, workspace, workspace_bytes, stream, nullptr,
                   0, false, &t);
}

kvs_status kvs_sparse_decode_attn_noalloc(const kvs_layout* L, int32_t table_kind, const void* q,
                                          const void* k_pool, const void* v_pool, const float* k_scales,
                                          const float* v_scales, const int32_t* table, const int32_t* seq_lens,
                                          const int32_t* sel, int32_t k, float sm_scale, float* out,
                                          void* stream) {
  return attn_impl(L, table_kind, q, k_pool, v_pool, k_scales, v_scales, table, seq_lens, sel, k, sm_scale, out,
                   nullptr, 0, stream, nullptr, 0, /*noalloc=*/true);
}

kvs_status kvs_score_blocks(const kvs_layout* L, const void* q, void* summaries, const int32_t* seq_lens,
                            const kvs_select_opts* opts, const kvs_append_args* append, double* scores,
                            double* bounds_out, void* stream) {
  if (!scores) return fail(KVS_ERR_INVALID_ARG, "scores must be non-NULL");
  SelectOpts o = opts_of(opts);
  o.recent = 1;  // not used here
  return select_impl(L, q, summaries, seq_lens, 0, nullptr, bounds_out, nullptr, 0, stream, nullptr, o, append,
                     scores);
}

kvs_status kvs_select_attn(const kvs_layout* L, const void* q, const void* k_pool, const void* v_pool,
                           const float* k_scales, const float* v_scales, const int32_t* block_table,
                           const int32_t* seq_lens, const double* scores, int32_t k, int32_t recent_blocks,
                           int32_t* sel, float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!scores || !aligned(scores, 8)) return fail(KVS_ERR_INVALID_ARG, "scores must be non-NULL and 8-byte aligned");
  if (k < 2 || (L && k > L->max_blocks)) return fail(KVS_ERR_INVALID_ARG, "k must be in [2, max_blocks]");
  if (recent_blocks < 1 || k < recent_blocks + 1)
    return fail(KVS_ERR_INVALID_ARG, "recent_blocks must be >= 1 and k >= recent_blocks + 1");
  return attn_impl(L, KVS_TABLE_PAGED, q, k_pool, v_pool, k_scales, v_scales, block_table, seq_lens, sel, k,
                   sm_scale, out, workspace, workspace_bytes, stream, scores, recent_blocks);
}

}  // extern "C"

namespace {

kvs_status attn_impl(const kvs_layout* L, int32_t table_kind, const void* q, const void* k_pool, const void* v_pool,
                     const float* k_scales, const float* v_scales, const int32_t* table, const int32_t* seq_lens,
                     const int32_t* sel, int32_t k, float sm_scale, float* out, void* workspace,
                     size_t workspace_bytes, void* stream, const double* scores, int32_t recent,
                     bool noalloc, const kvs::AppendArgs* tok) {
  // noalloc: the split partials go to the library's scratch array instead
  // of a caller's workspace (workspace and workspace_bytes are ignored)
  kvs_status st = check_layout(L, true);
  if (st != KVS_OK) return st;
  if (table_kind != KVS_TABLE_PAGED && table_kind != KVS_TABLE_HOT)
    return fail(KVS_ERR_INVALID_ARG, "unknown table_kind");
  if (!q || !k_pool || !v_pool || !table || !seq_lens || !sel || !out)
    return fail(KVS_ERR_INVALID_ARG, "q, pools, table, seq_lens, sel and out must be non-NULL");
  if (L->kv_dtype == KVS_FP8_E4M3 && (!k_scales || !v_scales))
    return fail(KVS_ERR_INVALID_ARG, "fp8 K/V need k_scales and v_scales");
  if (k < 1 || k > L->max_blocks) return fail(KVS_ERR_INVALID_ARG, "k must be in [1, max_blocks]");
  if (!(sm_scale == sm_scale) || sm_scale == __builtin_inff() || sm_scale == -__builtin_inff())
    return fail(KVS_ERR_INVALID_ARG, "sm_scale must be finite");
  if (noalloc) {
    const size_t need = attn_ws(L, k);
    if (need > kNoAllocScratchBytes)
      return fail(KVS_ERR_CAPACITY, "the split partials need " + std::to_string(need) +
                                        " bytes, more than KVS_NOALLOC_SCRATCH_BYTES (" +
                                        std::to_string(kNoAllocScratchBytes) + ")");
  } else if (!workspace || workspace_bytes < attn_ws(L, k)) {
    return fail(KVS_ERR_INVALID_ARG, "workspace missing or smaller than kvs_attn_workspace_size()");
  }
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || (!noalloc && !aligned(workspace, 16)) || !aligned(q, 4) ||
      !aligned(out, 4))
    return fail(KVS_ERR_INVALID_ARG, "pools and workspace must be 16-byte aligned");
  if (noalloc) {
    if ((st = scratch_ptr(&workspace)) != KVS_OK) return st;
    workspace_bytes = kNoAllocScratchBytes;
  }
  unsigned int* err = nullptr;
  if ((st = error_word(&err)) != KVS_OK) return st;
  kvs::AttnArgs a{};
  const int G = L->num_q_heads / L->num_kv_heads;
  const int nsplit = attn_splits(L, k);
  const size_t units = (size_t)L->num_seqs * L->num_q_heads * nsplit;
  char* ws = static_cast<char*>(workspace);
  a.part_m = reinterpret_cast<float*>(ws);
  a.part_l = a.part_m + units;
  a.part_acc = reinterpret_cast<float*>(ws + round_up(sizeof(float) * units * 2, 256));
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.table = table;
  a.seq_lens = seq_lens;
  a.sel = sel;
  a.out = out;
  a.err = err;
  a.q_scale = sm_scale * 1.4426950408889634f;
  a.B = L->num_seqs;
  a.Hq = L->num_q_heads;
  a.Hkv = L->num_kv_heads;
  a.G = G;
  a.D = L->head_dim;
  a.S = L->block_size;
  a.MB = L->max_blocks;
  a.P = L->num_pages;
  a.qg = L->quant_group;
  a.k = k;
  a.nsplit = nsplit;
  a.bps = (k + nsplit - 1) / nsplit;
  a.hot = table_kind == KVS_TABLE_HOT ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (scores) {
    if (kvs::attn_self_select_supported(kind_of(L->q_dtype), kind_of(L->kv_dtype), L->block_size, L->max_blocks, k)) {
      a.W = scores;  // each workgroup selects its own blocks
      a.sel_out = const_cast<int32_t*>(sel);
      a.recent = recent;
    } else {  // the attention kernel for this shape reads a selection: select first
      kvs::TopkArgs ta{};
      ta.W = scores;
      ta.seq_lens = seq_lens;
      ta.sel = const_cast<int32_t*>(sel);
      ta.B = L->num_seqs;
      ta.Hkv = L->num_kv_heads;
      ta.S = L->block_size;
      ta.MB = L->max_blocks;
      ta.k = k;
      ta.recent = recent;
      hipError_t e = kvs::launch_topk(ta, s);
      if (e != hipSuccess) return hip_status(e, "top-k launch");
    }
  }
  if (tok) {  // the token append first: in the same launch where the kernel allows, else its own
    kvs::AppendArgs t = *tok;
    t.err = err;
    if (kvs::attn_tok_supported(kind_of(L->q_dtype), kind_of(L->kv_dtype), L->block_size, L->head_dim, a.hot))
      return hip_status(kvs::launch_attn_tok(a, t, kind_of(L->q_dtype), kind_of(L->kv_dtype), s),
                        "append + attention launch");
    hipError_t e = kvs::launch_append(t, kind_of(L->kv_dtype), s);
    if (e != hipSuccess) return hip_status(e, "append launch");
  }
  return hip_status(kvs::launch_attn(a, kind_of(L->q_dtype), kind_of(L->kv_dtype), s), "attention launch");
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// The hot-buffer calls: `phases` = kvs::kHotLookup (page-table step, miss
// list) and/or kvs::kHotCopy (copy of the listed misses); the pointers a
// phase does not use may be NULL.
kvs_status hot_impl(const kvs_layout* L, const int32_t* sel, int32_t k, int32_t num_slots, int64_t step,
                    int32_t* page_table, int32_t* slot_owner, int64_t* slot_stamp, const void* host_k,
                    const void* host_v, const float* host_k_scales, const float* host_v_scales, void* hot_k,
                    void* hot_v, float* hot_k_scales, float* hot_v_scales, int32_t* miss_list,
                    int32_t* miss_count, const kvs_hot_live* live, void* stream, int phases) {
  const bool lookup = phases & kvs::kHotLookup, copy = phases & kvs::kHotCopy;
  kvs_status st = check_layout(L, false);
  if (st != KVS_OK) return st;
  if (!page_table || !miss_list || !miss_count || (lookup && (!sel || !slot_owner || !slot_stamp)) ||
      (copy && (!host_k || !host_v || !hot_k || !hot_v)))
    return fail(KVS_ERR_INVALID_ARG, "a required pointer is NULL");
  const bool fp8 = L->kv_dtype == KVS_FP8_E4M3;
  if (copy && fp8 && (!host_k_scales || !host_v_scales || !hot_k_scales || !hot_v_scales))
    return fail(KVS_ERR_INVALID_ARG, "fp8 pools need host and hot scales");
  if (num_slots < 1 || num_slots > 4096) return fail(KVS_ERR_UNSUPPORTED, "num_slots must be in [1, 4096]");
  if (k < 1 || k > L->max_blocks) return fail(KVS_ERR_INVALID_ARG, "k must be in [1, max_blocks]");
  if (k > num_slots) return fail(KVS_ERR_CAPACITY, "k selected blocks cannot fit in num_slots hot slots");
  if (step < 0 || step >= (1ll << 50)) return fail(KVS_ERR_INVALID_ARG, "step must be in [0, 2^50)");
  if ((long long)L->num_seqs * L->num_kv_heads * num_slots > 0x7FFFFFFFll)
    return fail(KVS_ERR_INVALID_ARG, "total hot slots overflow int32");
  if (copy && (!aligned(host_k, 16) || !aligned(host_v, 16) || !aligned(hot_k, 16) || !aligned(hot_v, 16)))
    return fail(KVS_ERR_INVALID_ARG, "host and hot pools must be 16-byte aligned");
  if (copy && live) {
    if (!live->k_pool || !live->v_pool || !live->block_table || !live->seq_lens ||
        (fp8 && (!live->k_scales || !live->v_scales)))
      return fail(KVS_ERR_INVALID_ARG, "live: pools, block_table and seq_lens (and fp8 scales) must be non-NULL");
    if (!aligned(live->k_pool, 16) || !aligned(live->v_pool, 16))
      return fail(KVS_ERR_INVALID_ARG, "live pools must be 16-byte aligned");
  }
  // device aliases of the pinned host tier (hipHostMalloc memory is mapped)
  const void* host_ptrs[4] = {host_k, host_v, host_k_scales, host_v_scales};
  void* dev_ptrs[4] = {nullptr, nullptr, nullptr, nullptr};
  for (int i = 0; copy && i < (fp8 ? 4 : 2); ++i) {
    hipError_t e = hipHostGetDevicePointer(&dev_ptrs[i], const_cast<void*>(host_ptrs[i]), 0);
    if (e != hipSuccess || !dev_ptrs[i]) {
      (void)hipGetLastError();
      return fail(KVS_ERR_INVALID_ARG, "host pools must be pinned host memory (hipHostMalloc)");
    }
  }
  unsigned int* err = nullptr;
  if ((st = error_word(&err)) != KVS_OK) return st;
  kvs::HotArgs a{};
  if (copy && live) {
    a.live_k = live->k_pool;
    a.live_v = live->v_pool;
    a.live_ks = fp8 ? live->k_scales : nullptr;
    a.live_vs = fp8 ? live->v_scales : nullptr;
    a.live_table = live->block_table;
    a.live_lens = live->seq_lens;
    a.P = L->num_pages;
  }
  a.sel = sel;
  a.pt = page_table;
  a.owner = slot_owner;
  a.stamp = slot_stamp;
  a.miss_list = miss_list;
  a.miss_count = miss_count;
  a.host_k = dev_ptrs[0];
  a.host_v = dev_ptrs[1];
  a.host_ks = static_cast<const float*>(dev_ptrs[2]);
  a.host_vs = static_cast<const float*>(dev_ptrs[3]);
  a.hot_k = hot_k;
  a.hot_v = hot_v;
  a.hot_ks = hot_k_scales;
  a.hot_vs = hot_v_scales;
  a.err = err;
  a.step = step;
  a.B = L->num_seqs;
  a.Hkv = L->num_kv_heads;
  a.D = L->head_dim;
  a.S = L->block_size;
  a.MB = L->max_blocks;
  a.k = k;
  a.ns = num_slots;
  int n2 = 1;
  while (n2 < num_slots) n2 <<= 1;
  a.n2 = n2 < 2 ? 2 : n2;
  a.qg = fp8 ? L->quant_group : 0;
  a.elem_bytes = (int)elem_size(L->kv_dtype);
  return hip_status(kvs::launch_hot(a, phases, static_cast<hipStream_t>(stream)), "hot-buffer launch");
}


}  // namespace

extern "C" {

kvs_status kvs_hot_lookup_swapin(const kvs_layout* L, const int32_t* sel, int32_t k, int32_t num_slots,
                                 int64_t step, int32_t* page_table, int32_t* slot_owner,
                                 int64_t* slot_stamp, const void* host_k, const void* host_v,
                                 const float* host_k_scales, const float* host_v_scales, void* hot_k,
                                 void* hot_v, float* hot_k_scales, float* hot_v_scales,
                                 int32_t* miss_list, int32_t* miss_count, const kvs_hot_live* live,
                                 void* stream) {
  return hot_impl(L, sel, k, num_slots, step, page_table, slot_owner, slot_stamp, host_k, host_v, host_k_scales,
                  host_v_scales, hot_k, hot_v, hot_k_scales, hot_v_scales, miss_list, miss_count, live, stream,
                  kvs::kHotLookup | kvs::kHotCopy);
}

kvs_status kvs_hot_lookup(const kvs_layout* L, const int32_t* sel, int32_t k, int32_t num_slots, int64_t step,
                          int32_t* page_table, int32_t* slot_owner, int64_t* slot_stamp, int32_t* miss_list,
                          int32_t* miss_count, void* stream) {
  return hot_impl(L, sel, k, num_slots, step, page_table, slot_owner, slot_stamp, nullptr, nullptr, nullptr,
                  nullptr, nullptr, nullptr, nullptr, nullptr, miss_list, miss_count, nullptr, stream,
                  kvs::kHotLookup);
}

kvs_status kvs_hot_swapin(const kvs_layout* L, int32_t k, int32_t num_slots, const int32_t* page_table,
                          const int32_t* miss_list, const int32_t* miss_count, const void* host_k,
                          const void* host_v, const float* host_k_scales, const float* host_v_scales,
                          void* hot_k, void* hot_v, float* hot_k_scales, float* hot_v_scales,
                          const kvs_hot_live* live, void* stream) {
  return hot_impl(L, nullptr, k, num_slots, 0, const_cast<int32_t*>(page_table), nullptr, nullptr, host_k, host_v,
                  host_k_scales, host_v_scales, hot_k, hot_v, hot_k_scales, hot_v_scales,
                  const_cast<int32_t*>(miss_list), const_cast<int32_t*>(miss_count), live, stream, kvs::kHotCopy);
}

}  // extern "C"
