// kvs_topk.h -- top-k selection of one (sequence, KV head) unit by a
// 256-thread workgroup (page "KV 稀疏化", §5 "Quest": keep the top-k blocks
// by score; the sink block and the R newest blocks are always kept, same
// page §2 and "SparDA：把KV選擇提前一層…" §4.2).  Used by topk_kernel and
// by the attention kernels that select their own blocks.
//
// The M = k-1-R best candidates (blocks 1..nb-R-1) under (W descending, id
// ascending) are found by bucket refinement.  A round takes the still
// undecided candidates, spreads them over 2048 LDS buckets by the monotone
// map (w - lo) * 2047 / (hi - lo) (lo, hi: their smallest and largest
// score), and scans the bucket counts from the top: candidates above the
// bucket where the count reaches the places left are taken, those below are
// dropped, and only that bucket's candidates stay undecided.  Those (at
// most 256 of them, else another round) are then ranked among themselves
// by (W desc, id asc) from a short LDS list, and the first ones fill the
// places left.  Rounds also end when the undecided candidates exactly fill
// the places left, or all hold one score (then the lowest ids win).  lo and
// hi always fall into different buckets, so every round decides at least
// one candidate; with real scores one round and the ranking settle the
// selection.  A block-wide prefix sum then writes the chosen ids in
// ascending order, then -1 padding.
//
// Cross-lane steps avoid LDS round trips: minima and maxima go through DPP
// row moves and readlane, prefix sums of small counts through one ballot and
// popcount per bit, and the bucket counts' prefix through a DPP scan; only
// the per-wavefront totals meet in LDS, behind one workgroup barrier each.
#pragma once

#include "kvs_internal.h"

namespace kvs {

constexpr int kTopkBuckets = 2048;
constexpr int kTopkList = 256;  // threshold-bucket candidates ranked directly

// LDS of one selection
struct TopkLds {
  unsigned hist[kTopkBuckets];
  double red_lo[4], red_hi[4];
  int scan_h[4], scan_c[4], scan_o[4];
  int sh_T, sh_rem, sh_all, sh_cnt, sh_len;
  double lw[kTopkList];
  int lid[kTopkList];
};

// One 32-bit DPP move inside a 16-lane row (CTRL: a permutation, so every
// lane has a source and `old` is never used).
template <int CTRL>
__device__ __forceinline__ double dpp_row_f64(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)((unsigned long long)b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane((int)(unsigned)b, lane);
  const int hi = __builtin_amdgcn_readlane((int)(unsigned)((unsigned long long)b >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Minimum (MAX = false) or maximum of x over the 64 lanes, in every lane:
// within each 16-lane row by DPP (lane pairs i^1, i^2, then the half-row and
// row mirrors), then the four rows' results by readlane.
template <bool MAX>
__device__ __forceinline__ double wave_minmax_f64(double x) {
  auto op = [](double a, double b) { return MAX ? fmax(a, b) : fmin(a, b); };
  x = op(x, dpp_row_f64<0xB1>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_row_f64<0x4E>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_row_f64<0x141>(x));  // row_half_mirror
  x = op(x, dpp_row_f64<0x140>(x));  // row_mirror
  return op(op(readlane_f64(x, 0), readlane_f64(x, 16)), op(readlane_f64(x, 32), readlane_f64(x, 48)));
}

// Exclusive prefix over the wavefront of a small non-negative v < 2^BITS,
// and the wavefront total, from one ballot per bit.
template <int BITS>
__device__ __forceinline__ int wave_prefix_small(int v, int* total) {
  const unsigned long long below = (1ull << (threadIdx.x & 63)) - 1ull;
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const unsigned long long m = __ballot((v >> b) & 1);
    pre += __popcll(m & below) << b;
    tot += __popcll(m) << b;
  }
  *total = tot;
  return pre;
}

// The same over the 256 threads (one workgroup barrier); `tmp` holds 4 ints
// of LDS that no other call uses before the next barrier.
template <int BITS>
__device__ __forceinline__ int block_prefix_small_256(int v, int* tmp, int* total) {
  const int wave = threadIdx.x >> 6;
  int wt;
  const int pre = wave_prefix_small<BITS>(v, &wt);
  if ((threadIdx.x & 63) == 0) tmp[wave] = wt;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = tmp[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + pre;
}

constexpr int bits_for(int n) { return n <= 1 ? 1 : 1 + bits_for(n / 2); }  // bits of values 0..n

// Inclusive prefix sum over the 64 lanes: DPP row shifts by 1, 2, 4 and 8
// within each 16-lane row (lanes shifted in from outside the row add 0),
// then lane 15's sum broadcast into row 1 and row 3, and lane 31's into rows
// 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive prefix over the 256 threads of any v >= 0, and the total, with
// six DPP steps per wavefront and one workgroup barrier (the wide counts of
// the bucket scan, where one ballot per bit would take 14 steps); `tmp` as
// for block_prefix_small_256.
__device__ __forceinline__ int block_prefix_256(int v, int* tmp, int* total) {
  const int wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if ((threadIdx.x & 63) == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = tmp[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + incl - v;
}

// min and max of the active scores and their count, over the 256 threads
// (one workgroup barrier)
template <int PT>
__device__ __forceinline__ void active_range(const double (&wv)[PT], const bool (&act)[PT], TopkLds& sh, double* lo,
                                             double* hi, int* n) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double l = __builtin_inf(), h = -__builtin_inf();
  int c = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    if (act[i]) {
      l = fmin(l, wv[i]);
      h = fmax(h, wv[i]);
    }
    c += __popcll(__ballot(act[i]));  // wavefront-uniform
  }
  l = wave_minmax_f64<false>(l);
  h = wave_minmax_f64<true>(h);
  if (lane == 0) {
    sh.red_lo[wave] = l;
    sh.red_hi[wave] = h;
    sh.scan_c[wave] = c;
  }
  __syncthreads();
  *lo = fmin(fmin(sh.red_lo[0], sh.red_lo[1]), fmin(sh.red_lo[2], sh.red_lo[3]));
  *hi = fmax(fmax(sh.red_hi[0], sh.red_hi[1]), fmax(sh.red_hi[2], sh.red_hi[3]));
  *n = sh.scan_c[0] + sh.scan_c[1] + sh.scan_c[2] + sh.scan_c[3];
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
  constexpr int CB = bits_for(PT);  // bits of a per-thread count 0..PT
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
      int before = block_prefix_small_256<CB>(c, sh.scan_o, &tot);
#pragma unroll
      for (int i = 0; i < PT; ++i)
        if (act[i]) {
          take[i] = take[i] || before < need;
          ++before;
        }
      __syncthreads();  // scan_o is read again by the output scan below
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
    int above = block_prefix_256(s, sh.scan_h, &tot);
    if (above < need && need <= above + s) {  // exactly one thread
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (above + (int)cnt[q] >= need) {
          sh.sh_T = kTopkBuckets - 1 - BPT * tid - q;
          sh.sh_rem = need - above;
          sh.sh_all = above + (int)cnt[q] == need;  // the bucket fills the places exactly
          sh.sh_cnt = (int)cnt[q];
          sh.sh_len = 0;
          break;
        }
        above += (int)cnt[q];
      }
    }
    __syncthreads();
    const int T = sh.sh_T;
    need = sh.sh_rem;
    const bool all = sh.sh_all != 0;
    const int cnt_T = sh.sh_cnt;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      take[i] = take[i] || bk[i] > T || (all && bk[i] == T);
      act[i] = act[i] && bk[i] == T;
    }
    if (all) break;
    if (cnt_T <= kTopkList) {
      // rank the threshold bucket's candidates among themselves by (W desc,
      // id asc): the `need` first ones are taken
#pragma unroll
      for (int i = 0; i < PT; ++i)
        if (act[i]) {
          const int slot = (int)atomicAdd((unsigned*)&sh.sh_len, 1u);
          if (slot < kTopkList) {  // always: exactly cnt_T candidates append
            sh.lw[slot] = wv[i];
            sh.lid[slot] = j0 + i;
          }
        }
      __syncthreads();
      const int m = min(cnt_T, kTopkList);
      int rank[PT];
#pragma unroll
      for (int i = 0; i < PT; ++i) rank[i] = 0;
      bool any = false;
#pragma unroll
      for (int i = 0; i < PT; ++i) any = any || act[i];
      if (any) {
        for (int e = 0; e < m; ++e) {
          const double w = sh.lw[e];
          const int id = sh.lid[e];
#pragma unroll
          for (int i = 0; i < PT; ++i) rank[i] += (w > wv[i] || (w == wv[i] && id < j0 + i)) ? 1 : 0;
        }
      }
#pragma unroll
      for (int i = 0; i < PT; ++i) take[i] = take[i] || (act[i] && rank[i] < need);
      break;
    }
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
  int pos = block_prefix_small_256<CB>(n_sel, sh.scan_o, &tot);
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if ((chosen & (1u << i)) && pos < k) out[pos++] = j0 + i;
  for (int i = tot + tid; i < k; i += 256) out[i] = -1;
}

}  // namespace kvs
