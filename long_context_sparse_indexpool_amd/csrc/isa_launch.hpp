// isa_launch.hpp -- host-side launchers of the gfx950 kernels (internal to libisa).
#pragma once

#include <hip/hip_ext.h>

#include "isa_common.hpp"

namespace isa {

// Compute units and XCDs (chiplets with their own L2) of the calling thread's
// current device, queried once per device and cached.  Workgroups are
// dispatched round-robin over the XCDs, which the attention and prefill
// launches use to place workgroups that share data on one L2; the decode
// scoring tile size follows the CU count.
struct DevInfo {
  int n_cu;
  int n_xcd;
};
DevInfo device_info();

constexpr int TILE_G = 8192;      // pooled groups of the largest decode work tile (128 pages)
constexpr int TILE_SKEW_MAX = 320;  // groups a tile of a pair may take over from its partner (5 pages)
constexpr int TILE_CAP = TILE_G + TILE_SKEW_MAX;  // candidates one tile can emit: the list stride
constexpr int TILE_G_MIN = 2048;  // smallest tile, for batches that would not fill the chip
constexpr int TILE_MAX_PER_SEQ = (ISA_MAX_SEQ_LEN / GROUP + TILE_G - 1) / TILE_G;

constexpr int PAIR_CAP = NBINS;  // (bin, count) pairs a decode tile can emit

// Decode indexer workspace (pointers into the caller's workspace).
struct DecodeWs {
  uint32_t* err;
  uint2* tile_meta;      // [ntiles] (candidates kept, pairs)
  uint32_t* tile_pairs;  // [ntiles][PAIR_CAP]
  uint64_t* tile_list;   // [ntiles][TILE_CAP]
};

isa_status launch_indexer_decode(const BatchArgs& a, const int8_t* q, const int8_t* hw, const int8_t* pooled,
                                 const int32_t* bt, const DecodeWs& w, int32_t* out_idx, int32_t* out_count,
                                 int32_t* scores_out, int32_t ld_scores, hipStream_t stream);

isa_status launch_topk_rows(const int32_t* scores, int32_t rows, int32_t cols, int32_t ld, int32_t k,
                            int32_t* out_idx, int32_t* out_count, hipStream_t stream);

isa_status launch_indexpool(const BatchArgs& a, const uint16_t* keys, const float w4[4], const int32_t* bt,
                            float* scales, int8_t* pooled, bool dynamic, float* amax_part, uint32_t* err,
                            hipStream_t stream);
constexpr int POOL_TILE_G = 256;  // groups per pooling work tile (4 pages)
isa_status launch_append(const BatchArgs& a, const uint16_t* key_new, const uint16_t* latent_new, const float w4[4],
                         const int32_t* bt, const float* scales, uint16_t* keys, uint16_t* latent, int8_t* pooled,
                         uint32_t* err, hipStream_t stream);

// Sparse MLA attention: split plan chosen on the host.
struct MlaPlan {
  int32_t rows;
  int32_t splits;         // token splits per row
  int32_t groups_per_split;
};
struct MlaWs {
  uint32_t* err;
  char* o_part;     // [layers][rows][splits][64] slots of 2 KiB: a head's normalised partial O / l,
                    // 512 fp16 values (first KiB) or 512 fp32 values
  float* ml_part;   // [layers][rows][splits][64][4]: reference (log2 units), sum, format (1 = fp32), 0
};
MlaPlan plan_mla(int32_t rows, int32_t k, int32_t layers);
// n_layers (1..ISA_MAX_LAYERS) attentions that share one selection; q, latent,
// out are host arrays of n_layers device pointers, lse null or such an array.
// lat_scale null: latent rows are bf16; otherwise the rows are FP8 E4M3 codes
// and lat_scale an array of n_layers per-row scale pools.
isa_status launch_sparse_mla(const BatchArgs& a, const MlaPlan& p, int32_t n_layers, const uint16_t* const* q,
                             const void* const* latent, const float* const* lat_scale, const int32_t* bt,
                             const int32_t* row_seq,
                             const int32_t* row_pos, const int32_t* idx, const int32_t* count, int32_t k,
                             float sm_scale, float* const* out, float* const* lse, const MlaWs& w,
                             hipStream_t stream);

isa_status launch_latent_fp8(const BatchArgs& a, const uint16_t* latent, const int32_t* bt, uint8_t* codes,
                             float* scales, uint32_t* err, hipStream_t stream);

isa_status launch_kda_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                           const float* beta, uint16_t* state, float* out, int32_t n, uint32_t* err,
                           hipStream_t stream);

isa_status launch_prefill_scores(const BatchArgs& a, const int8_t* q, const int8_t* hw, const int32_t* q_pos,
                                 int32_t Q, const int8_t* pooled, const int32_t* bt, int32_t* scores,
                                 int32_t ld, uint32_t* err, hipStream_t stream);

isa_status launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// Benchmark timing hook (isa_set_kernel_timer): a ring of event pairs that the
// dispatch itself records (hipExtLaunchKernelGGL), so the elapsed time is the
// kernel's own execution.
constexpr int TIMER_MAX = 4096;
struct KernelTimer {
  int n = 0, next = 0;
  hipEvent_t start[TIMER_MAX], stop[TIMER_MAX];
};
extern KernelTimer g_timer[3];
template <class Kernel, class... Args>
hipError_t launch_timed(int timer, Kernel kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  KernelTimer& t = g_timer[timer];
  if (t.n) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t.start[t.next], t.stop[t.next], 0, args...);
    t.next = (t.next + 1) % t.n;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  }
  return hipGetLastError();
}

}  // namespace isa
