// kvs_topk.h -- top-k selection of one (sequence, KV head) unit by a
// 256-thread workgroup (page "KV 稀疏化", §5 "Quest": keep the top-k blocks
// by score; the sink block and the R newest blocks are always kept, same
// page §2 and "SparDA：把KV選擇提前一層…" §4.2).  Used by topk_kernel and
// by the attention kernels that select their own blocks.
//
// The M = k-1-R best candidates (blocks 1..nb-R-1) under (W descending, id
// ascending) are found by bucket refinement.  Each round takes the still
// undecided candidates, spreads them over 2048 LDS buckets by the monotone
// map (w - lo) * 2047 / (hi - lo) (lo, hi: their smallest and largest
// score), and scans the bucket counts from the top: candidates above the
// bucket where the count reaches the places left are taken, those below are
// dropped, and only that bucket's candidates stay undecided.  The rounds end
// when the undecided candidates exactly fill the places left, or when they
// all hold one score (then the lowest ids win).  lo and hi always fall into
// different buckets, so every round decides at least one candidate; with
// real scores one or two rounds settle the selection.  A block-wide prefix
// sum then writes the chosen ids in ascending order, then -1 padding.
#pragma once

#include "kvs_internal.h"

namespace kvs {

constexpr int kTopkBuckets = 2048;

// LDS of one selection
struct TopkLds {
  unsigned hist[kTopkBuckets];
  double red_lo[4], red_hi[4];
  int red_n[4];
  int scan_tmp[4];
  int sh_T, sh_rem, sh_all;
};

// min and max of the active scores and their count, over the 256 threads
// (one workgroup barrier)
template <int PT>
__device__ __forceinline__ void active_range(const double (&wv)[PT], const bool (&act)[PT], TopkLds& sh, double* lo,
                                             double* hi, int* n) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double l = __builtin_inf(), h = -__builtin_inf();
  int c = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if (act[i]) {
      l = fmin(l, wv[i]);
      h = fmax(h, wv[i]);
      ++c;
    }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    l = fmin(l, __shfl_xor(l, off));
    h = fmax(h, __shfl_xor(h, off));
    c += __shfl_xor(c, off);
  }
  if (lane == 0) {
    sh.red_lo[wave] = l;
    sh.red_hi[wave] = h;
    sh.red_n[wave] = c;
  }
  __syncthreads();
  *lo = fmin(fmin(sh.red_lo[0], sh.red_lo[1]), fmin(sh.red_lo[2], sh.red_lo[3]));
  *hi = fmax(fmax(sh.red_hi[0], sh.red_hi[1]), fmax(sh.red_hi[2], sh.red_hi[3]));
  *n = sh.red_n[0] + sh.red_n[1] + sh.red_n[2] + sh.red_n[3];
}

// A unit's scores W[0..MB): thread t holds ids t*per .. t*per+per-1,
// per = ceil(MB/256) <= PT.  Ids past the unit's block count are loaded but
// never used.
template <int PT>
__device__ __forceinline__ void load_unit_scores(const double* W, int MB, double (&wv)[PT]) {
  const int per = (MB + 255) / 256;
  const int j0 = (int)threadIdx.x * per;
#pragma unroll
  for (int i = 0; i < PT; ++i) wv[i] = (i < per && j0 + i < MB) ? W[j0 + i] : 0.0;
}

// The selection of a unit with nb blocks into out[0..k): if nb <= k every
// block, else block 0, blocks nb-R..nb-1 and the k-1-R best of the others.
// Every thread of the 256-thread workgroup calls it; out may be global or
// LDS memory (the caller synchronises before reading it back).
template <int PT>
__device__ __forceinline__ void select_unit(const double (&wv)[PT], int MB, int nb, int k, int R, int32_t* out,
                                            TopkLds& sh) {
  const int tid = threadIdx.x;
  const int per = (MB + 255) / 256;
  const int j0 = tid * per;
  if (nb <= k) {  // every block, then padding
    for (int i = tid; i < k; i += 256) out[i] = i < nb ? i : -1;
    return;
  }
  // nb > k >= R + 1: the sink and the window do not meet
  bool act[PT], take[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    act[i] = i < per && j >= 1 && j < nb - R;  // candidates
    take[i] = false;
  }
  int need = k - 1 - R;  // places left for undecided candidates
  constexpr int BPT = kTopkBuckets / 256;  // buckets per thread
  for (;;) {  // every round decides at least one candidate
    // the round's histogram is cleared here; active_range's barrier orders
    // the clear before the counting below
#pragma unroll
    for (int q = 0; q < BPT; ++q) sh.hist[q * 256 + tid] = 0u;
    double lo, hi;
    int n;
    active_range<PT>(wv, act, sh, &lo, &hi, &n);
    // (lo, hi, n and need are the same in every thread: the exits are uniform)
    if (need == 0) break;
    if (n <= need) {  // the undecided candidates fill the places left
#pragma unroll
      for (int i = 0; i < PT; ++i) take[i] = take[i] || act[i];
      break;
    }
    if (!(lo < hi)) {  // one score left: the lowest ids win
      int c = 0;
#pragma unroll
      for (int i = 0; i < PT; ++i) c += act[i] ? 1 : 0;
      int tot;
      int before = block_exclusive_scan_256(c, sh.scan_tmp, &tot);
#pragma unroll
      for (int i = 0; i < PT; ++i)
        if (act[i]) {
          take[i] = take[i] || before < need;
          ++before;
        }
      break;
    }
    // bucket of each undecided candidate, nondecreasing in its score: lo in
    // bucket 0, hi in the last bucket
    const double scale = (double)(kTopkBuckets - 1) / (hi - lo);
    int bk[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const double x = (wv[i] - lo) * scale;
      int v = -1;
      if (act[i]) v = wv[i] == lo ? 0 : (wv[i] == hi || !(x < kTopkBuckets - 1) ? kTopkBuckets - 1 : (int)x);
      bk[i] = v;
    }
#pragma unroll
    for (int i = 0; i < PT; ++i)
      if (bk[i] >= 0) atomicAdd(&sh.hist[bk[i]], 1u);
    __syncthreads();
    // thread t sums buckets last-BPT*t down to last-BPT*t-(BPT-1) (from the top)
    unsigned cnt[BPT];
    int s = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      cnt[q] = sh.hist[kTopkBuckets - 1 - BPT * tid - q];
      s += (int)cnt[q];
    }
    int tot;
    int above = block_exclusive_scan_256(s, sh.scan_tmp, &tot);
    if (above < need && need <= above + s) {  // exactly one thread
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (above + (int)cnt[q] >= need) {
          sh.sh_T = kTopkBuckets - 1 - BPT * tid - q;
          sh.sh_rem = need - above;
          sh.sh_all = above + (int)cnt[q] == need;  // the bucket fills the places exactly
          break;
        }
        above += (int)cnt[q];
      }
    }
    __syncthreads();
    const int T = sh.sh_T;
    need = sh.sh_rem;
    const bool all = sh.sh_all != 0;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      take[i] = take[i] || bk[i] > T || (all && bk[i] == T);
      act[i] = act[i] && bk[i] == T;
    }
    if (all) break;
  }
  // ascending output: the sink, the chosen candidates, the window
  int n_sel = 0;
  unsigned chosen = 0u;  // bit i: id j0+i selected
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    if (i >= per || j >= nb) continue;
    if (j == 0 || j >= nb - R || take[i]) {
      chosen |= 1u << i;
      ++n_sel;
    }
  }
  int tot;
  int pos = block_exclusive_scan_256(n_sel, sh.scan_tmp, &tot);
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if ((chosen & (1u << i)) && pos < k) out[pos++] = j0 + i;
  for (int i = tot + tid; i < k; i += 256) out[i] = -1;
}

}  // namespace kvs
