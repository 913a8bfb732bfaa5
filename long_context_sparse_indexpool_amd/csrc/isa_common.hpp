// isa_common.hpp -- constants, launch arguments and device helpers shared by the
// gfx950 kernels of the IndexPool sparse-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/isa.h"

namespace isa {

// Fixed dimensions of the path (see isa.h).
constexpr int IDX_DIM = 128;     // indexer key / query channels
constexpr int IDX_HEADS = 32;    // lightning-indexer heads
constexpr int GROUP = 4;         // tokens pooled into one indexer key
constexpr int ATT_HEADS = 64;    // MLA query heads
constexpr int LAT_DIM = 512;     // MLA latent width (keys = values)
constexpr int PAGE_TOK = 256;    // tokens per page
constexpr int PAGE_GRP = PAGE_TOK / GROUP;  // pooled groups per page
constexpr int MAX_K = ISA_MAX_K;

// Score histogram: a monotone 11-bit key of a 32-bit score (exact below 128,
// then 64 sub-bins per octave).  Used by every top-k kernel.
constexpr int NBINS = 2048;
constexpr uint32_t INVALID_SCORE = 0xFFFFFFFFu;  // never a valid score (max valid < 2^32 - 1)

__device__ __forceinline__ int score_bin(uint32_t s) {
  if (s < 64u) return (int)s;
  int e = 31 - __clz(s);  // 6..31
  return ((e - 5) << 6) | (int)((s >> (e - 6)) & 63u);
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// Per-call description of the batch, passed by value in the kernel arguments so
// that no host-to-device copy is needed: lengths and a tile prefix per sequence.
struct BatchArgs {
  int32_t batch;
  int32_t max_pages;
  int32_t num_pages;
  int32_t k;
  int32_t tile_g;  // pooled groups per decode scoring tile (a multiple of 64, 2048 .. 8192)
  int32_t tile_skew;  // groups the even-numbered tile of a full pair takes over from the odd one (see k_indexer_score)
  int32_t lens[ISA_MAX_BATCH];
  int32_t tile_start[ISA_MAX_BATCH + 1];  // first work tile of each sequence
};

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt 0) and meets the other waves, without the workgroup memory fence of
// __syncthreads(), whose release part also waits for every outstanding global
// load -- which would drain register prefetches at each barrier.  Use it only
// where the barrier orders LDS accesses, not global ones.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt/expcnt at maximum (no wait), lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Sticky device error word (first word of every workspace).
__device__ __forceinline__ void report(uint32_t* err, uint32_t bits) {
  if (err) atomicOr(err, bits);
}

// Physical page of logical page j of sequence b, or -1 (and an error bit) when
// the block table points outside the pool.
__device__ __forceinline__ int phys_page(const int32_t* __restrict__ bt, int max_pages, int num_pages, int b,
                                         int j, uint32_t* err) {
  int p = bt[(size_t)b * max_pages + j];
  if (p < 0 || p >= num_pages) {
    report(err, ISA_DERR_PAGE_OOB);
    return -1;
  }
  return p;
}

// Sequence owning work tile `t`: the number of sequences whose first tile is
// <= t, minus one.  Each lane of the wave tests one sequence (one round of
// loads from the argument block instead of a chain of dependent ones) and a
// ballot counts them.  The result is uniform across the wave.
__device__ __forceinline__ int tile_owner(const BatchArgs& a, int t) {
  const int lane = threadIdx.x & 63;
  int n = 0;
#pragma unroll
  for (int base = 0; base < ISA_MAX_BATCH; base += 64) {
    if (base < a.batch) {
      const bool le = base + lane < a.batch && a.tile_start[base + lane] <= t;
      n += __popcll(__ballot(le));
    }
  }
  return n - 1;
}

// Inclusive prefix sum across a 64-lane wave with DPP moves: shifts of 1, 2, 4
// and 8 lanes inside each row of 16, then row broadcasts 15 and 31 carry the
// row totals upward (lanes whose source is outside the range add 0).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum over the lanes of one wave; *total receives the wave's
// sum (the same in every lane).
__device__ __forceinline__ uint32_t wave_exclusive_scan(uint32_t v, uint32_t* total) {
  const uint32_t x = wave_inclusive_scan(v);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
  return x - v;
}

// Block-wide exclusive prefix sum of one value per thread (blockDim.x <= 1024,
// a multiple of 64).  `tmp` holds >= blockDim.x/64 + 1 words of LDS.  Returns
// the exclusive prefix; *total receives the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  if (threadIdx.x < 64) {  // scan of the wave totals by the first wave
    uint32_t t = threadIdx.x < nw ? tmp[threadIdx.x] : 0u;
    uint32_t it = wave_inclusive_scan(t);
    if (threadIdx.x < nw) tmp[threadIdx.x] = it - t;
    if (threadIdx.x == nw - 1) tmp[nw] = it;
  }
  __syncthreads();
  const uint32_t r = tmp[wid] + x - v;
  *total = tmp[nw];
  __syncthreads();
  return r;
}

}  // namespace isa
