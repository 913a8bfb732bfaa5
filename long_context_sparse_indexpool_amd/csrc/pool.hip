// pool.hip -- IndexPool and int8 quantisation of the indexer key cache, gfx950.
//
// Method (pages cited by title): "GLM-5.3-Flash: 하이브리드 희소·선형 어텐션과
// IndexPool·EPD로 1M 컨텍스트를 오픈 소스로 서빙하는 방법" (llm-wiki.hwlabs.dev),
// section "IndexPool: 인덱서 KV 캐시를 4배 압축": four consecutive indexer keys merge
// into one, k_pool = sum_i w_i k_i with learned weights summing to 1, which
// quarters the cache; section "양자화: W8A8와 혼합 캐시": the distant compressed
// cache is kept in INT8.  The quantiser (not on the pages): one symmetric
// scale per sequence, amax/127, round half to even, clamp to +-127.  A last
// group of r < 4 tokens renormalises its r weights.
//
// HBM-bound stream: 1 KiB of bf16 keys in, 128 B of int8 out per group.  A
// workgroup handles 256 groups (4 key pages) of one sequence; 16 threads per
// group, 8 channels each, 16-byte loads and 8-byte stores.  The dynamic scale
// needs the sequence's amax first: a first launch writes per-tile maxima, and
// every workgroup of the second launch reduces its sequence's maxima (a few
// KiB, from L2) before it pools again and quantises; the kernel boundary
// makes the maxima visible, with no fence or ticket (on this 8-XCD part a
// device-scope release per workgroup writes back the L2 and costs more than
// the stream).  A given scale skips the first pass.
#include "isa_launch.hpp"

namespace isa {

constexpr int POOL_THREADS = 256;
constexpr int POOL_ITERS = POOL_TILE_G / (POOL_THREADS / 16);

struct PoolPtrs {
  const uint16_t* keys;
  const int32_t* bt;
  float* scales;
  int8_t* pooled;
  float* amax_part;   // [ntiles]
  uint32_t* err;
  float w[4];
};

// k_pool passes: per-tile maxima; quantise with the given scales; quantise
// with the scales of the maxima (and write them)
enum PoolMode { POOL_AMAX = 0, POOL_GIVEN = 1, POOL_DYNAMIC = 2 };

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Pooled fp32 values of channels 8c..8c+7 of group g (r tokens present).
// With `last` given, token r - 1 is taken from it instead of from memory.
__device__ __forceinline__ void pool8(const float (&wt)[4], const uint16_t* grp, int r, int c, float (&x)[8],
                                      const v4i* last = nullptr) {
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.f;
  float wsum = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t < r) {
      v4i v = (last && t == r - 1) ? *last : *reinterpret_cast<const v4i*>(grp + t * IDX_DIM + c * 8);
      const float w = wt[t];
      wsum += w;
      x[0] = fmaf(w, bf16_lo(v.x), x[0]);
      x[1] = fmaf(w, bf16_hi(v.x), x[1]);
      x[2] = fmaf(w, bf16_lo(v.y), x[2]);
      x[3] = fmaf(w, bf16_hi(v.y), x[3]);
      x[4] = fmaf(w, bf16_lo(v.z), x[4]);
      x[5] = fmaf(w, bf16_hi(v.z), x[5]);
      x[6] = fmaf(w, bf16_lo(v.w), x[6]);
      x[7] = fmaf(w, bf16_hi(v.w), x[7]);
    }
  }
  if (r < 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = x[i] / wsum;
  }
}

// Eight pooled values quantised with `scale`: round half to even, clamp to
// +-127, packed little-endian.
__device__ __forceinline__ uint2 quant8(const float (&x)[8], float scale) {
  uint32_t packed[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float qv = __builtin_rintf(x[i] / scale);  // round half to even
    qv = fminf(fmaxf(qv, -127.f), 127.f);
    packed[i >> 2] |= ((uint32_t)((int32_t)qv) & 0xFFu) << (8 * (i & 3));
  }
  return make_uint2(packed[0], packed[1]);
}

template <int MODE>
__global__ __launch_bounds__(POOL_THREADS) void k_pool(const BatchArgs a, const PoolPtrs P) {
  constexpr bool QUANT = MODE != POOL_AMAX;
  __shared__ int32_t pages[POOL_TILE_G / PAGE_GRP];
  __shared__ float red[POOL_THREADS / 64];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int b = tile_owner(a, tile);
  const int t0 = a.tile_start[b];
  const int L = a.lens[b];
  const int G = (L + GROUP - 1) / GROUP;
  const int g0 = (tile - t0) * POOL_TILE_G;
  if (tid < POOL_TILE_G / PAGE_GRP) {
    int j = g0 / PAGE_GRP + tid;
    pages[tid] = (g0 + tid * PAGE_GRP < G) ? phys_page(P.bt, a.max_pages, a.num_pages, b, j, P.err) : -1;
  }
  float scale = 1.f;
  if (MODE == POOL_DYNAMIC) {  // the sequence's amax from the first launch's per-tile maxima
    const int ntiles = a.tile_start[b + 1] - t0;
    float m = 0.f;
    for (int i = tid; i < ntiles; i += POOL_THREADS) m = fmaxf(m, P.amax_part[t0 + i]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((tid & 63) == 0) red[tid >> 6] = m;
  }
  __syncthreads();
  const int c = tid & 15;  // channel block
  if (MODE == POOL_DYNAMIC) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < POOL_THREADS / 64; ++i) m = fmaxf(m, red[i]);
    scale = m > 0.f ? m / 127.f : 1.f;
    if (tile == t0 && tid == 0) P.scales[b] = scale;
    if (!isfinite(scale)) scale = 1.f;  // an infinite key: already reported by the first pass
  } else if (MODE == POOL_GIVEN) {
    scale = P.scales[b];
    if (!(scale > 0.f) || !isfinite(scale)) {
      if (tid == 0) report(P.err, ISA_DERR_NONFINITE);
      scale = 1.f;
    }
  }
  float amax = 0.f;
  bool nonfinite = false;
  for (int it = 0; it < POOL_ITERS; ++it) {
    const int gl = it * (POOL_THREADS / 16) + (tid >> 4);
    const int g = g0 + gl;
    if (g >= G) break;
    const int pg = pages[gl / PAGE_GRP];
    if (pg < 0) continue;
    const int r = min(4, L - 4 * g);
    const uint16_t* grp = P.keys + ((size_t)pg * PAGE_TOK + (size_t)(4 * g) % PAGE_TOK) * IDX_DIM;
    float x[8];
    pool8(P.w, grp, r, c, x);
    if (QUANT) {
      int8_t* dst = P.pooled + ((size_t)pg * PAGE_GRP + g % PAGE_GRP) * IDX_DIM + c * 8;
      *reinterpret_cast<uint2*>(dst) = quant8(x, scale);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        nonfinite |= !isfinite(x[i]);
        amax = fmaxf(amax, fabsf(x[i]));
      }
    }
  }
  if (QUANT) return;

  // ---- per-tile amax ----
  if (__any(nonfinite) && (tid & 63) == 0) report(P.err, ISA_DERR_NONFINITE);
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  if (tid == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < POOL_THREADS / 64; ++i) m = fmaxf(m, red[i]);
    P.amax_part[tile] = m;
  }
}

// Decode-time append: one 64-thread workgroup per sequence writes the new
// token (position L - 1) into the key and latent pools and re-pools its group
// from the r tokens now present, with the same arithmetic as k_pool, so the
// result equals a full re-pool at the given scale.  Threads 0..15 own 8 key
// channels each; all 64 copy 16 B of the latent row.  The new key enters the
// pooling from registers; the group's earlier tokens come from earlier calls.
struct AppendPtrs {
  const uint16_t* key_new;
  const uint16_t* latent_new;
  const int32_t* bt;
  const float* scales;
  uint16_t* keys;
  uint16_t* latent;
  int8_t* pooled;
  uint32_t* err;
  float w[4];
};

__global__ __launch_bounds__(64) void k_append(const BatchArgs a, const AppendPtrs A) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int t = a.lens[b] - 1;  // the new token
  const int pg = phys_page(A.bt, a.max_pages, a.num_pages, b, t / PAGE_TOK, A.err);
  if (pg < 0) return;
  const size_t row = (size_t)pg * PAGE_TOK + t % PAGE_TOK;
  if (A.latent_new) {
    const v4i v = reinterpret_cast<const v4i*>(A.latent_new + (size_t)b * LAT_DIM)[tid];
    reinterpret_cast<v4i*>(A.latent + row * LAT_DIM)[tid] = v;
  }
  if (tid >= IDX_DIM / 8) return;
  const v4i k = reinterpret_cast<const v4i*>(A.key_new + (size_t)b * IDX_DIM)[tid];
  reinterpret_cast<v4i*>(A.keys + row * IDX_DIM)[tid] = k;
  const int g = t / GROUP, r = t % GROUP + 1;
  float scale = A.scales[b];
  if (!(scale > 0.f) || !isfinite(scale)) {
    if (tid == 0) report(A.err, ISA_DERR_NONFINITE);
    scale = 1.f;
  }
  const uint16_t* grp = A.keys + ((size_t)pg * PAGE_TOK + (size_t)(4 * g) % PAGE_TOK) * IDX_DIM;
  float x[8];
  pool8(A.w, grp, r, tid, x, &k);
  *reinterpret_cast<uint2*>(A.pooled + ((size_t)pg * PAGE_GRP + g % PAGE_GRP) * IDX_DIM + tid * 8) = quant8(x, scale);
}

isa_status launch_append(const BatchArgs& a, const uint16_t* key_new, const uint16_t* latent_new, const float w4[4],
                         const int32_t* bt, const float* scales, uint16_t* keys, uint16_t* latent, int8_t* pooled,
                         uint32_t* err, hipStream_t stream) {
  AppendPtrs A{key_new, latent_new, bt, scales, keys, latent, pooled, err, {w4[0], w4[1], w4[2], w4[3]}};
  hipLaunchKernelGGL(k_append, dim3(a.batch), dim3(64), 0, stream, a, A);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

isa_status launch_indexpool(const BatchArgs& a, const uint16_t* keys, const float w4[4], const int32_t* bt,
                            float* scales, int8_t* pooled, bool dynamic, float* amax_part, uint32_t* err,
                            hipStream_t stream) {
  const int ntiles = a.tile_start[a.batch];
  PoolPtrs P{keys, bt, scales, pooled, amax_part, err, {w4[0], w4[1], w4[2], w4[3]}};
  if (dynamic) {
    hipLaunchKernelGGL(k_pool<POOL_AMAX>, dim3(ntiles), dim3(POOL_THREADS), 0, stream, a, P);
    if (hipGetLastError() != hipSuccess) return ISA_ERR_HIP;
    hipLaunchKernelGGL(k_pool<POOL_DYNAMIC>, dim3(ntiles), dim3(POOL_THREADS), 0, stream, a, P);
  } else {
    hipLaunchKernelGGL(k_pool<POOL_GIVEN>, dim3(ntiles), dim3(POOL_THREADS), 0, stream, a, P);
  }
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

}  // namespace isa
