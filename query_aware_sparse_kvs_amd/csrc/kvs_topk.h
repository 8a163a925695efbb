// kvs_topk.h -- top-k selection of one (sequence, KV head) unit by a
// 256-thread workgroup (page "KV 稀疏化", §5 "Quest": keep the top-k blocks
// by score; the sink block and the R newest blocks are always kept, same
// page §2 and "SparDA：把KV選擇提前一層…" §4.2).  Used by topk_kernel and
// by the attention kernels that select their own blocks.
//
// Scores are mapped to order-preserving 64-bit keys.  A most-significant-digit
// radix select (8-bit digits, LDS histogram) over the high 32 bits, starting
// at the first bit where the candidates' keys differ, finds the bucket of the
// (k-1-R)-th largest key among blocks 1..nb-R-1; only when that bucket holds
// more keys than are needed does a second select run on the low 32 bits of
// the tied keys.  Ties on the full key go to the lowest block ids, the
// (W desc, id asc) order.  A block-wide prefix sum writes the chosen ids in
// ascending order, then -1 padding.
#pragma once

#include "kvs_internal.h"

namespace kvs {

// order-preserving map of a double (no NaN) to uint64; -0 and +0 coincide
__device__ __forceinline__ unsigned long long order_key(double w) {
  const double z = w + 0.0;  // -0 -> +0
  const unsigned long long u = (unsigned long long)__double_as_longlong(z);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Radix select over the active 32-bit keys of a 256-thread workgroup: finds
// the value T of the rem-th largest active key (rem is 1-based) and how many
// keys equal to T are needed (*rem_eq).  Keys share the bits above byte
// `start_byte` (given in `prefix`), so only bytes start_byte..0 are scanned.
template <int PT>
__device__ __forceinline__ void radix_select_u32(const unsigned (&key)[PT], const bool (&act)[PT], int rem,
                                                 int start_byte, unsigned prefix, unsigned* hist,
                                                 unsigned* sh_T, int* sh_rem, unsigned* T, int* rem_eq) {
  const int tid = threadIdx.x;
  unsigned mask = start_byte >= 3 ? 0u : (0xFFFFFFFFu << (8 * (start_byte + 1)));
  prefix &= mask;
  for (int pass = start_byte; pass >= 0; --pass) {
    const int shift = pass * 8;
    hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PT; ++i)
      if (act[i] && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 255-4l .. 252-4l (highest digits first)
      unsigned c4[4], s = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = hist[255 - 4 * tid - e];
        s += c4[e];
      }
      unsigned incl = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned o = __shfl_up(incl, off);
        if (tid >= off) incl += o;
      }
      unsigned above = incl - s;  // keys in higher digits
      if ((int)above < rem && rem <= (int)incl) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((int)(above + c4[e]) >= rem) {
            *sh_T = prefix | ((unsigned)(255 - 4 * tid - e) << shift);
            *sh_rem = rem - (int)above;
            break;
          }
          above += c4[e];
        }
      }
    }
    __syncthreads();
    prefix = *sh_T;
    rem = *sh_rem;
    mask |= 0xFFu << shift;
  }
  *T = prefix;
  *rem_eq = rem;
}

// block-wide min and max of v over 256 threads (tmp: 8 words of LDS)
__device__ __forceinline__ void block_min_max_256(unsigned v_min, unsigned v_max, unsigned* tmp, unsigned* mn,
                                                  unsigned* mx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    v_min = min(v_min, (unsigned)__shfl_xor((int)v_min, off));
    v_max = max(v_max, (unsigned)__shfl_xor((int)v_max, off));
  }
  if (lane == 0) {
    tmp[wave] = v_min;
    tmp[4 + wave] = v_max;
  }
  __syncthreads();
  *mn = min(min(tmp[0], tmp[1]), min(tmp[2], tmp[3]));
  *mx = max(max(tmp[4], tmp[5]), max(tmp[6], tmp[7]));
}

// LDS of one selection
struct TopkLds {
  unsigned hist[256];
  unsigned mm_tmp[8];
  int scan_tmp[4];
  unsigned sh_T;
  int sh_rem;
};

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
  const int M = k - 1 - R;  // free picks among blocks 1..nb-R-1

  bool cand[PT];
  unsigned hi[PT], lo[PT];
  unsigned hmin = 0xFFFFFFFFu, hmax = 0u;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    cand[i] = i < per && j >= 1 && j < nb - R;
    const unsigned long long key = cand[i] ? order_key(wv[i]) : 0ull;
    hi[i] = (unsigned)(key >> 32);
    lo[i] = (unsigned)key;
    if (cand[i]) {
      hmin = min(hmin, hi[i]);
      hmax = max(hmax, hi[i]);
    }
  }
  // phase 1: threshold on the high 32 bits of the key
  unsigned T_hi = 0u, T_lo = 0u;
  int rem_hi = 0, rem_lo = 0, n_eq = 0;
  bool need_lo = false;
  bool eqh[PT];
  if (M > 0) {
    unsigned mn, mx;
    block_min_max_256(hmin, hmax, sh.mm_tmp, &mn, &mx);
    if (mn == mx) {
      T_hi = mn;
      rem_hi = M;
    } else {
      const int top_bit = 31 - __clz(mn ^ mx);
      radix_select_u32<PT>(hi, cand, M, top_bit / 8, mn, sh.hist, &sh.sh_T, &sh.sh_rem, &T_hi, &rem_hi);
    }
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      eqh[i] = cand[i] && hi[i] == T_hi;
      cnt += eqh[i] ? 1 : 0;
    }
    int tot;
    (void)block_exclusive_scan_256(cnt, sh.scan_tmp, &tot);
    n_eq = tot;
    // phase 2 (only when the threshold bucket holds more keys than needed):
    // threshold on the low 32 bits among the keys tied on the high bits
    need_lo = rem_hi < n_eq;
    if (need_lo) {
      unsigned lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
      for (int i = 0; i < PT; ++i)
        if (eqh[i]) {
          lmin = min(lmin, lo[i]);
          lmax = max(lmax, lo[i]);
        }
      unsigned mn2, mx2;
      block_min_max_256(lmin, lmax, sh.mm_tmp, &mn2, &mx2);
      if (mn2 == mx2) {
        T_lo = mn2;
        rem_lo = rem_hi;
      } else {
        const int top_bit = 31 - __clz(mn2 ^ mx2);
        radix_select_u32<PT>(lo, eqh, rem_hi, top_bit / 8, mn2, sh.hist, &sh.sh_T, &sh.sh_rem, &T_lo, &rem_lo);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PT; ++i) eqh[i] = false;
  }
  // ties on the full key go to the lowest block ids
  int n_tie = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) n_tie += (need_lo && eqh[i] && lo[i] == T_lo) ? 1 : 0;
  int tot;
  int tie_before = block_exclusive_scan_256(n_tie, sh.scan_tmp, &tot);
  int n_sel = 0;
  unsigned chosen = 0u;  // bit i: id j0+i selected
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int j = j0 + i;
    if (i >= per || j >= nb) continue;
    bool take;
    if (j == 0 || j >= nb - R) {
      take = true;
    } else if (!cand[i] || M == 0) {
      take = false;
    } else if (hi[i] != T_hi) {
      take = hi[i] > T_hi;
    } else if (!need_lo) {
      take = true;  // the whole bucket is needed
    } else if (lo[i] != T_lo) {
      take = lo[i] > T_lo;
    } else {
      take = tie_before < rem_lo;
      ++tie_before;
    }
    if (take) {
      chosen |= 1u << i;
      ++n_sel;
    }
  }
  int pos = block_exclusive_scan_256(n_sel, sh.scan_tmp, &tot);
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if ((chosen & (1u << i)) && pos < k) out[pos++] = j0 + i;
  for (int i = tot + tid; i < k; i += 256) out[i] = -1;
}

}  // namespace kvs
