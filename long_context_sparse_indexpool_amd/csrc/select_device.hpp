// select_device.hpp -- block-level building blocks of the exact top-k selection.
//
// The order is "higher score first, then lower group id".  Scores are unsigned
// 32-bit; a candidate's composite key (score << 32) | (0xFFFFFFFF - id) is
// unique and larger exactly when the candidate ranks higher, so selecting the m
// largest composite keys realises the tie rule.
#pragma once

#include "isa_common.hpp"

namespace isa {

__device__ __forceinline__ uint64_t rank_key(uint32_t score, uint32_t id) {
  return ((uint64_t)score << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }
__device__ __forceinline__ uint32_t key_score(uint64_t key) { return (uint32_t)(key >> 32); }

// Appends the lanes whose pred holds to a list with one LDS atomic per wave:
// returns this lane's slot (the wave's base plus its rank among the appending
// lanes).  Every lane of the wave calls it.
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const unsigned long long mask = __ballot(pred);
  const uint32_t n = (uint32_t)__popcll(mask);
  uint32_t base = 0;
  if ((threadIdx.x & 63) == 0 && n) base = atomicAdd(counter, n);
  base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
  return base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// LDS scratch layout used below: words [0, 17) by block_exclusive_scan, results
// at RES.. .
constexpr int SCR_WORDS = 64;
constexpr int SCR_RES = 40;

// hist[NBINS] in LDS.  Finds the highest bin `bstar` whose suffix count (bins
// >= bstar) reaches K; *n_gt = count of bins above it.  If the total is below
// K, *bstar = -1 and *n_gt = total.  All threads must call; results are
// uniform.
__device__ __forceinline__ void find_boundary(const uint32_t* hist, uint32_t K, int* bstar, uint32_t* n_gt,
                                              uint32_t* total, uint32_t* scr) {
  const int per = NBINS / (int)blockDim.x;
  const int hi = NBINS - (int)threadIdx.x * per;  // this thread owns bins [hi - per, hi)
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) local += hist[hi - 1 - j];
  uint32_t tot;
  uint32_t above = block_exclusive_scan(local, scr, &tot);
  if (threadIdx.x == 0 && tot < K) {
    scr[SCR_RES] = 0xFFFFFFFFu;
    scr[SCR_RES + 1] = tot;
  }
  if (tot >= K && above < K && above + local >= K) {
    uint32_t run = above;
    for (int j = 0; j < per; ++j) {
      int bin = hi - 1 - j;
      uint32_t c = hist[bin];
      if (run + c >= K) {
        scr[SCR_RES] = (uint32_t)bin;
        scr[SCR_RES + 1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  *bstar = (int)scr[SCR_RES];
  *n_gt = scr[SCR_RES + 1];
  *total = tot;
  __syncthreads();
}

// Exact threshold of the top-m composite keys among a candidate set that
// `each(f)` enumerates (every thread calls f(key) for the candidates it owns;
// the set must be the same on every call).  Returns the m-th largest key, so
// the selected candidates are exactly those with key >= the result.
// h256: 256 words of LDS.  m >= 1 and m <= |set|.
template <class Each>
__device__ uint64_t radix_select_threshold(Each each, uint32_t m, uint32_t* h256, uint32_t* scr) {
  uint64_t prefix = 0, mask = 0;
  uint32_t rem = m;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) h256[i] = 0;
    __syncthreads();
    each([&](uint64_t key) {
      if ((key & mask) == prefix) atomicAdd(&h256[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    uint32_t c = threadIdx.x < 256 ? h256[255 - threadIdx.x] : 0u;
    uint32_t tot;
    uint32_t above = block_exclusive_scan(c, scr, &tot);
    if (threadIdx.x < 256 && above < rem && above + c >= rem) {
      scr[SCR_RES + 2] = 255u - threadIdx.x;
      scr[SCR_RES + 3] = above;
    }
    __syncthreads();
    uint32_t d = scr[SCR_RES + 2];
    rem -= scr[SCR_RES + 3];
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    __syncthreads();
  }
  return prefix;
}

// Ascending bitonic sort of n (a power of two, <= 1024) words in LDS.
__device__ __forceinline__ void bitonic_sort_asc(uint32_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint32_t x = a[i], y = a[ixj];
          bool up = (i & k) == 0;
          if ((x > y) == up) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
}

// Sort `n` selected ids held in sel[0..n) ascending and write a row of the
// output (k entries, -1 padded) plus its count.
__device__ __forceinline__ void write_sorted_row(uint32_t* sel, int n, int k, int32_t* out_idx_row,
                                                 int32_t* out_count_row) {
  for (int i = n + threadIdx.x; i < MAX_K; i += blockDim.x) sel[i] = 0xFFFFFFFFu;
  __syncthreads();
  bitonic_sort_asc(sel, MAX_K);
  for (int i = threadIdx.x; i < k; i += blockDim.x) out_idx_row[i] = i < n ? (int32_t)sel[i] : -1;
  if (threadIdx.x == 0) *out_count_row = n;
}

}  // namespace isa
