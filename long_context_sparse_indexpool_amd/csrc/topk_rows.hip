// topk_rows.hip -- exact top-k selection over rows of precomputed int32 scores
// (the prefill path: one row per query), for gfx950.
//
// Selection rule (pages cited by title): "GLM-5.3 Sparse Attention은 연산량을 줄이지만
// HBM 수요는 지속된다" (remio.ai), section "GLM-5.3 Sparse Attention이 실제로 바꾸는
// 것": keep the top-k positions; with no more than k candidates nothing is
// dropped.  Ties (unspecified on the pages): higher score first, then lower id.
//
// One 1024-thread workgroup per row, no workspace; rows are streamed with 16-B
// loads, several in flight per thread.  Pass 1 streams the row into
// an LDS histogram over the 11-bit monotone score key and finds the bin holding
// the k-th best.  Pass 2 streams it again: ids above that bin are selected
// outright, ids in it become (score, -id) keys in LDS (or, when they do not
// fit, are re-enumerated from the row), and an 8-bit radix select resolves the
// remaining slots exactly.  The k ids are sorted ascending in LDS and written.
#include "isa_launch.hpp"
#include "select_device.hpp"

namespace isa {

constexpr int ROW_THREADS = 1024;
constexpr int ROW_CAND = 2048;
constexpr int ROW_UNROLL = 4;  // 16-B loads of a thread in flight per round

// f(score, id) for every entry of the row, in any order.  A 16-B aligned row
// (the usual case: ld a multiple of 4) is read with 16-B loads, ROW_UNROLL of
// them issued by each thread before any is used (entries past the row read as
// -1, which every caller skips); otherwise entry by entry.
template <class F>
__device__ __forceinline__ void for_each_entry(const int32_t* __restrict__ row, int32_t cols, bool aligned, F&& f) {
  const int tid = threadIdx.x;
  if (aligned) {
    const int4* row4 = reinterpret_cast<const int4*>(row);
    const int n4 = cols >> 2;
    for (int i0 = 0; i0 < n4; i0 += ROW_UNROLL * ROW_THREADS) {
      int4 v[ROW_UNROLL];
#pragma unroll
      for (int u = 0; u < ROW_UNROLL; ++u) v[u] = row4[min(i0 + u * ROW_THREADS + tid, n4 - 1)];
#pragma unroll
      for (int u = 0; u < ROW_UNROLL; ++u) {
        const int i = i0 + u * ROW_THREADS + tid;
        const int4 w = i < n4 ? v[u] : make_int4(-1, -1, -1, -1);  // masked at use, not at load
        f(w.x, 4 * i);
        f(w.y, 4 * i + 1);
        f(w.z, 4 * i + 2);
        f(w.w, 4 * i + 3);
      }
    }
    for (int e = 4 * n4 + tid; e < cols; e += ROW_THREADS) f(row[e], e);
  } else {
    for (int e = tid; e < cols; e += ROW_THREADS) f(row[e], e);
  }
}

__global__ __launch_bounds__(ROW_THREADS) void k_topk_rows(const int32_t* __restrict__ scores, int32_t cols,
                                                           int32_t ld, int32_t k, int32_t* __restrict__ out_idx,
                                                           int32_t* __restrict__ out_count) {
  __shared__ uint32_t hist[NBINS];
  __shared__ uint64_t cand[ROW_CAND];
  __shared__ uint32_t sel[MAX_K];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t scr[SCR_WORDS];
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const uint32_t K = (uint32_t)k;
  const int32_t* row = scores + (size_t)r * ld;
  int32_t* orow = out_idx + (size_t)r * k;

  const bool aligned = ((uintptr_t)row & 15u) == 0;  // uniform
  for (int i = tid; i < NBINS; i += ROW_THREADS) hist[i] = 0;
  __syncthreads();
  for_each_entry(row, cols, aligned, [&](int32_t s, int) {
    if (s >= 0) atomicAdd(&hist[score_bin((uint32_t)s)], 1u);
  });
  __syncthreads();
  int bstar;
  uint32_t n_gt, total;
  find_boundary(hist, K, &bstar, &n_gt, &total, scr);

  if (bstar < 0) {  // at most k candidates: all of them, in id order
    uint32_t base = 0;
    for (int e0 = 0; e0 < cols; e0 += ROW_THREADS) {
      int e = e0 + tid;
      uint32_t v = (e < cols && row[e] >= 0) ? 1u : 0u;
      uint32_t tot;
      uint32_t pos = block_exclusive_scan(v, scr, &tot);
      if (v) orow[base + pos] = e;
      base += tot;
    }
    for (int i = (int)base + tid; i < k; i += ROW_THREADS) orow[i] = -1;
    if (tid == 0) out_count[r] = (int32_t)base;
    return;
  }

  const uint32_t m = K - n_gt;
  if (tid == 0) {
    scr[SCR_RES + 10] = 0;
    scr[SCR_RES + 11] = 0;
  }
  __syncthreads();
  for_each_entry(row, cols, aligned, [&](int32_t s, int e) {
    if (s < 0) return;
    int bin = score_bin((uint32_t)s);
    if (bin > bstar) {
      uint32_t p = atomicAdd(&scr[SCR_RES + 10], 1u);
      if (p < MAX_K) sel[p] = (uint32_t)e;
    } else if (bin == bstar) {
      uint32_t p = atomicAdd(&scr[SCR_RES + 11], 1u);
      if (p < ROW_CAND) cand[p] = rank_key((uint32_t)s, (uint32_t)e);
    }
  });
  __syncthreads();
  const uint32_t nb = scr[SCR_RES + 11];
  const bool in_lds = nb <= ROW_CAND;
  uint64_t thr;
  if (in_lds) {
    thr = radix_select_threshold(
        [&](auto f) {
          for (uint32_t i = tid; i < nb; i += ROW_THREADS) f(cand[i]);
        },
        m, h256, scr);
  } else {
    thr = radix_select_threshold(
        [&](auto f) {
          for (int e = tid; e < cols; e += ROW_THREADS) {
            int32_t s = row[e];
            if (s >= 0 && score_bin((uint32_t)s) == bstar) f(rank_key((uint32_t)s, (uint32_t)e));
          }
        },
        m, h256, scr);
  }
  if (tid == 0) scr[SCR_RES + 12] = 0;
  __syncthreads();
  if (in_lds) {
    for (uint32_t i = tid; i < nb; i += ROW_THREADS)
      if (cand[i] >= thr) {
        uint32_t p = n_gt + atomicAdd(&scr[SCR_RES + 12], 1u);
        if (p < MAX_K) sel[p] = key_id(cand[i]);
      }
  } else {
    for (int e = tid; e < cols; e += ROW_THREADS) {
      int32_t s = row[e];
      if (s >= 0 && score_bin((uint32_t)s) == bstar && rank_key((uint32_t)s, (uint32_t)e) >= thr) {
        uint32_t p = n_gt + atomicAdd(&scr[SCR_RES + 12], 1u);
        if (p < MAX_K) sel[p] = (uint32_t)e;
      }
    }
  }
  __syncthreads();
  write_sorted_row(sel, (int)K, k, orow, out_count + r);
}

isa_status launch_topk_rows(const int32_t* scores, int32_t rows, int32_t cols, int32_t ld, int32_t k,
                            int32_t* out_idx, int32_t* out_count, hipStream_t stream) {
  hipLaunchKernelGGL(k_topk_rows, dim3(rows), dim3(ROW_THREADS), 0, stream, scores, cols, ld, k, out_idx,
                     out_count);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

}  // namespace isa
