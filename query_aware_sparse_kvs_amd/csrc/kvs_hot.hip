// kvs_hot.hip -- hot-buffer page-table step and swap-in copy (page
// "KV 稀疏化", §7 "HiSparse": a hot device buffer holds the KV the current
// top-k set is likely to touch, inactive KV sits in host memory, and a
// swap-in step on the decode path finds the misses, updates the page table
// and copies the KV back; what stays resident follows the selection).
//
// hot_lookup_kernel: one 256-thread workgroup per (sequence, KV head) unit.
//   1. stage and check the selection row (ascending ids then -1) and the
//      unit's owner table; mark the selected ids in an LDS bitmap;
//   2. hits refresh their slot's stamp; misses are compacted in ascending
//      order with a block prefix sum (miss list + count);
//   3. every slot whose owner is not selected gets the key
//      (stamp+1) << 13 | slot, every other slot the largest key; a bitonic
//      sort in LDS orders them, so the r-th smallest is the r-th victim;
//   4. the r-th miss takes the r-th victim (old owner unmapped).
//   Integer work only; latency-bound.
// swapin_copy_kernel: two workgroups per unit, each copying every other
//   miss's K and V tiles (and fp8 scales) from pinned host memory into its
//   hot slot with 16-byte loads, a tile's loads all issued before its
//   stores; with a live cache, the unit's newest block (still receiving
//   tokens, never in the host tier whole) comes from the device pool, hit
//   or miss.  Bound by the host link.
#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kSlotBits = 13;  // slot ids < 8192

__global__ __launch_bounds__(256) void hot_lookup_kernel(HotArgs a) {
  extern __shared__ unsigned long long hkeys[];  // [n2]
  __shared__ int sh_n, sh_bad, scan_tmp[4];
  const int u = blockIdx.x, tid = threadIdx.x;
  const int k = a.k, ns = a.ns, MB = a.MB;
  const int32_t* srow = a.sel + (long long)u * k;
  int32_t* pt = a.pt + (long long)u * MB;
  int32_t* owner = a.owner + (long long)u * ns;
  int64_t* stamp = a.stamp + (long long)u * ns;
  int32_t* mlist = a.miss_list + (long long)u * k;
  const int base = u * ns;
  // bitmap of selected ids lives in the tail of the key buffer
  unsigned int* inS = reinterpret_cast<unsigned int*>(hkeys + a.n2);
  const int words = (MB + 31) / 32;

  if (tid == 0) {
    sh_n = k;
    sh_bad = 0;
  }
  for (int w = tid; w < words; w += 256) inS[w] = 0u;
  __syncthreads();
  for (int i = tid; i < k; i += 256)
    if (srow[i] == -1) atomicMin(&sh_n, i);
  __syncthreads();
  const int n = sh_n;
  for (int i = tid; i < k; i += 256) {
    const int j = srow[i];
    bool bad;
    if (i < n)
      bad = j < 0 || j >= MB || (i > 0 && srow[i - 1] >= j);
    else
      bad = j != -1;
    if (bad) atomicOr(&sh_bad, 0x4);
    else if (i < n) atomicOr(&inS[j >> 5], 1u << (j & 31));
  }
  // owner table and the page-table entries of the selected ids must agree
  for (int s = tid; s < ns; s += 256) {
    const int o = owner[s];
    if (o != -1 && (o < 0 || o >= MB || pt[o] != base + s)) atomicOr(&sh_bad, 0x2);
  }
  for (int i = tid; i < n; i += 256) {
    const int j = srow[i];
    if (j < 0 || j >= MB) continue;
    const int p = pt[j];
    if (p != -1 && (p < base || p >= base + ns || owner[p - base] != j)) atomicOr(&sh_bad, 0x2);
  }
  __syncthreads();
  if (sh_bad) {
    if (tid == 0) {
      raise_flag(a.err, (unsigned)sh_bad);
      a.miss_count[u] = 0;
    }
    for (int i = tid; i < k; i += 256) mlist[i] = -1;
    return;
  }

  // hits and misses (ids in ascending order; each thread takes a run)
  const int per = (n + 255) / 256;
  const int i0 = tid * per;
  int n_miss = 0;
  for (int q = 0; q < per; ++q) {
    const int i = i0 + q;
    if (i >= n) break;
    const int p = pt[srow[i]];
    if (p >= 0)
      stamp[p - base] = a.step;
    else
      ++n_miss;
  }
  int m;
  int pos = block_exclusive_scan_256(n_miss, scan_tmp, &m);
  for (int q = 0; q < per; ++q) {
    const int i = i0 + q;
    if (i >= n) break;
    const int j = srow[i];
    if (pt[j] < 0) mlist[pos++] = j;
  }
  for (int i = m + tid; i < k; i += 256) mlist[i] = -1;
  if (tid == 0) a.miss_count[u] = m;

  // victim order: (stamp asc, slot asc) among slots not holding a selected id
  for (int s = tid; s < a.n2; s += 256) {
    unsigned long long key = ~0ull;
    if (s < ns) {
      const int o = owner[s];
      const bool held = o >= 0 && ((inS[o >> 5] >> (o & 31)) & 1u);
      if (!held) key = ((unsigned long long)(stamp[s] + 1) << kSlotBits) | (unsigned long long)s;
    }
    hkeys[s] = key;
  }
  __syncthreads();
  for (int size = 2; size <= a.n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int x = tid; x < (a.n2 >> 1); x += 256) {
        const int lo = 2 * x - (x & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned long long kl = hkeys[lo], kh = hkeys[hi];
        if ((kl > kh) == up) {
          hkeys[lo] = kh;
          hkeys[hi] = kl;
        }
      }
      __syncthreads();
    }
  }
  // miss r -> victim r; the miss list was written by this workgroup above
  __threadfence_block();
  for (int r = tid; r < m; r += 256) {
    if (hkeys[r] == ~0ull) continue;  // cannot happen after the checks above
    const int s = (int)(hkeys[r] & ((1ull << kSlotBits) - 1));
    const int j = mlist[r];
    const int old = owner[s];
    if (old >= 0) pt[old] = -1;
    pt[j] = base + s;
    owner[s] = j;
    stamp[s] = a.step;
  }
}

// Copy workgroups per unit: each takes every kCopyGroups-th block to copy.
// Few workgroups suffice to keep the host link busy (two tiles of 16 KiB per
// workgroup in flight), and they leave most SIMDs free for kernels that run
// beside the copy (the attention of another layer).
constexpr int kCopyGroups = 2;

// One tile (K, V, and fp8 scales) copied by a workgroup, 16-byte vectors.
__device__ __forceinline__ void copy_tile(const HotArgs& a, const char* sk, const char* sv, const float* ssk,
                                          const float* ssv, long long slot, long long tile_bytes) {
  const int tid = threadIdx.x;
  const int n16 = (int)(tile_bytes / 16);
  constexpr int kMaxPer = 8;  // 16-byte vectors per thread per round
  const u32x4* k16 = reinterpret_cast<const u32x4*>(sk);
  const u32x4* v16 = reinterpret_cast<const u32x4*>(sv);
  u32x4* dk = reinterpret_cast<u32x4*>(static_cast<char*>(a.hot_k) + slot * tile_bytes);
  u32x4* dv = reinterpret_cast<u32x4*>(static_cast<char*>(a.hot_v) + slot * tile_bytes);
  for (int x0 = 0; x0 < n16; x0 += 256 * kMaxPer) {
    u32x4 bk[kMaxPer], bv[kMaxPer];
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
      const int x = x0 + q * 256 + tid;
      bk[q] = bv[q] = u32x4{0u, 0u, 0u, 0u};
      if (x < n16) {
        bk[q] = k16[x];
        bv[q] = v16[x];
      }
    }
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
      const int x = x0 + q * 256 + tid;
      if (x < n16) {
        dk[x] = bk[q];
        dv[x] = bv[q];
      }
    }
  }
  if (a.qg > 0) {
    const int ns_per_tile = a.S * (a.D / a.qg);
    float* dsk = a.hot_ks + slot * ns_per_tile;
    float* dsv = a.hot_vs + slot * ns_per_tile;
    for (int x = tid; x < ns_per_tile; x += 256) {
      dsk[x] = ssk[x];
      dsv[x] = ssv[x];
    }
  }
}

// The unit's misses, in list order, come from the host tier.  With a live
// cache the unit's newest block comes from it instead: as a miss (then it is
// the list's last entry, misses being ascending and the newest block the
// highest id a selection holds) or, when it is resident anyway, as one more
// item.  (A selection holding ids past the sequence can list it earlier; it
// is then copied twice, from the same source.)
__global__ __launch_bounds__(256) void swapin_copy_kernel(HotArgs a) {
  const int u = blockIdx.y, tid = threadIdx.x;
  int m = a.miss_count[u];
  m = m < 0 ? 0 : (m > a.k ? a.k : m);  // miss_list holds k entries per unit
  const long long tile_bytes = (long long)a.S * a.D * a.elem_bytes;
  const int ns_per_tile = a.qg > 0 ? a.S * (a.D / a.qg) : 0;
  const int b = u / a.Hkv, g = u % a.Hkv;
  int newest = -1;  // the unit's newest block, taken from the live cache
  int items = m;
  if (a.live_k) {
    int len = a.live_lens[b];
    const int cap = a.MB * a.S;
    if (len < 0 || len > cap) {
      if (tid == 0 && blockIdx.x == 0 && g == 0) raise_flag(a.err, 0x1u);
      len = len < 0 ? 0 : cap;
    }
    newest = len > 0 ? (len - 1) / a.S : -1;
    const bool listed = m > 0 && a.miss_list[(long long)u * a.k + m - 1] == newest;
    if (newest >= 0 && !listed && a.pt[(long long)u * a.MB + newest] >= 0) items = m + 1;
  }
  for (int r = blockIdx.x; r < items; r += kCopyGroups) {  // items is uniform over the workgroup
    const int j = r < m ? a.miss_list[(long long)u * a.k + r] : newest;
    if (j < 0 || j >= a.MB) continue;
    const int slot = a.pt[(long long)u * a.MB + j];
    if (slot < u * a.ns || slot >= (u + 1) * a.ns) {
      if (tid == 0) raise_flag(a.err, 0x2u);
      continue;
    }
    if (j == newest) {  // from the live cache
      const int page = a.live_table[(long long)b * a.MB + j];
      if (page < 0 || page >= a.P) {
        if (tid == 0) raise_flag(a.err, 0x2u);
        continue;
      }
      const long long t = (long long)page * a.Hkv + g;
      copy_tile(a, static_cast<const char*>(a.live_k) + t * tile_bytes,
                static_cast<const char*>(a.live_v) + t * tile_bytes, a.live_ks + t * ns_per_tile,
                a.live_vs + t * ns_per_tile, slot, tile_bytes);
    } else {  // from the host tier
      const long long t = (long long)u * a.MB + j;
      copy_tile(a, static_cast<const char*>(a.host_k) + t * tile_bytes,
                static_cast<const char*>(a.host_v) + t * tile_bytes, a.host_ks + t * ns_per_tile,
                a.host_vs + t * ns_per_tile, slot, tile_bytes);
    }
  }
}

}  // namespace

hipError_t launch_hot(const HotArgs& a, int phases, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int units = a.B * a.Hkv;
  if (phases & kHotLookup) {
    const size_t lds = sizeof(unsigned long long) * (size_t)a.n2 + sizeof(unsigned int) * (size_t)((a.MB + 31) / 32);
    hipLaunchKernelGGL(hot_lookup_kernel, dim3((unsigned)units), dim3(256), lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kHotCopy)
    hipLaunchKernelGGL(swapin_copy_kernel, dim3((unsigned)kCopyGroups, (unsigned)units), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvs
