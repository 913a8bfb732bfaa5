// api.hip -- the C ABI of libisa (see include/isa.h): argument validation on
// the host, workspace layout, work plans passed by value to the kernels, and
// launches on the caller's stream.  Nothing here allocates or synchronises
// except isa_device_error, which reads the error word on request.
#include <string.h>

#include <mutex>

#include "isa_launch.hpp"

namespace isa {
namespace {

// Workspace layout shared by every call: the sticky error word in the first
// 256 bytes, then the call's own scratch, which every kernel writes before it
// reads it within the same call -- nothing in it has to survive between calls,
// so a workspace can be reused for any batch shape or shared between calls.
constexpr size_t HDR = 256;
constexpr size_t SCR0 = HDR;

inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline int64_t groups_of(int32_t L) { return ((int64_t)L + GROUP - 1) / GROUP; }

// Host validation of a batch description.
bool valid_seqs(const isa_seqs* s) {
  if (!s || s->batch < 1 || s->batch > ISA_MAX_BATCH || s->max_pages < 1 || s->num_pages < 1 || s->reserved != 0 ||
      !s->seq_lens_host || !s->block_table || !aligned16(s->block_table))
    return false;
  for (int b = 0; b < s->batch; ++b) {
    int32_t L = s->seq_lens_host[b];
    if (L < 1 || L > ISA_MAX_SEQ_LEN) return false;
    if ((L + PAGE_TOK - 1) / PAGE_TOK > s->max_pages) return false;
  }
  return true;
}

void fill_batch(const isa_seqs* s, BatchArgs* a, int32_t k) {
  memset(a, 0, sizeof(*a));
  a->batch = s->batch;
  a->max_pages = s->max_pages;
  a->num_pages = s->num_pages;
  a->k = k;
  a->tile_g = TILE_G;
  for (int b = 0; b < s->batch; ++b) a->lens[b] = s->seq_lens_host[b];
}

// Groups the even-numbered tile of a full pair takes over from its odd
// partner.  Workgroups are dispatched round-robin over the XCDs, so tile
// parity is XCD parity; on this part the even XCDs stream their tiles about 8%
// faster than the odd ones (per-workgroup timelines of the scoring kernel,
// every workload measured), so an even tile gets about 4% more groups: whole
// pages, 5 of 128 for the largest tiles.  No skew when the XCD count is odd.
int32_t decode_tile_skew(int32_t tg) {
  if ((device_info().n_xcd & 1) != 0) return 0;
  return tg * TILE_SKEW_MAX / TILE_G / PAGE_GRP * PAGE_GRP;  // 320 for tiles of 8192, 128 at 4096 .. 6528, 64 below
}

int decode_tiles(int32_t L, int32_t k, int32_t tg) {
  int64_t G = groups_of(L);
  return G <= k ? 1 : (int)((G + tg - 1) / tg);
}

// Pooled groups per decode scoring tile.  8192 when that already gives at
// least one tile per CU.  Otherwise the smallest multiple of PAGE_GRP, at
// least TILE_G_MIN, whose tiles fit in one round over the CUs: a batch that
// would make slightly more tiles than CUs runs them all at once, each a little
// larger, instead of leaving a second round of tiles to a few CUs while the
// rest wait (halving the tile to reach one tile per CU could double the
// kernel).  Every sequence stays within the tiles per sequence the selection
// handles, which 8192 always satisfies.  The tile count does not depend on k
// (every tile holds more than MAX_K groups), so the workspace query and the
// call agree.
int32_t decode_tile_g(const isa_seqs* s) {
  const int N_CU = device_info().n_cu;
  auto fits = [&](int32_t tg) {
    int nt = 0;
    for (int b = 0; b < s->batch; ++b) {
      const int t = decode_tiles(s->seq_lens_host[b], MAX_K, tg);
      if (t > TILE_MAX_PER_SEQ) return false;
      nt += t;
    }
    return nt <= N_CU;
  };
  int nt_max = 0;
  for (int b = 0; b < s->batch; ++b) nt_max += decode_tiles(s->seq_lens_host[b], MAX_K, TILE_G);
  if (nt_max >= N_CU) return TILE_G;
  // the tile count only falls as tiles grow: the smallest fitting multiple
  int32_t lo = TILE_G_MIN / PAGE_GRP, hi = TILE_G / PAGE_GRP;  // in pages; hi fits
  if (fits(lo * PAGE_GRP)) return TILE_G_MIN;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) / 2;
    if (fits(mid * PAGE_GRP))
      hi = mid;
    else
      lo = mid;
  }
  return hi * PAGE_GRP;
}

int pool_tiles(int32_t L) { return (int)((groups_of(L) + POOL_TILE_G - 1) / POOL_TILE_G); }

struct DecodeLayout {
  size_t tile_meta, tile_pairs, tile_list, total;
};
DecodeLayout decode_layout(const isa_seqs* s, int32_t k) {
  DecodeLayout d;
  const int32_t tg = decode_tile_g(s);
  int nt = 0;
  for (int b = 0; b < s->batch; ++b) nt += decode_tiles(s->seq_lens_host[b], k, tg);
  d.tile_meta = SCR0;
  d.tile_pairs = d.tile_meta + up256((size_t)nt * 8);
  d.tile_list = d.tile_pairs + up256((size_t)nt * PAIR_CAP * 4);
  d.total = d.tile_list + up256((size_t)nt * TILE_CAP * 8);
  return d;
}

size_t pool_ws(const isa_seqs* s) {
  int nt = 0;
  for (int b = 0; b < s->batch; ++b) nt += pool_tiles(s->seq_lens_host[b]);
  return SCR0 + up256((size_t)nt * 4);  // per-tile maxima of the dynamic scale
}

size_t mla_ws(int32_t rows, int32_t k, int32_t layers) {
  MlaPlan p = plan_mla(rows, k, layers);
  if (p.splits <= 1) return HDR;
  return SCR0 + up256((size_t)layers * rows * p.splits * ATT_HEADS * LAT_DIM * 4) +
         up256((size_t)layers * rows * p.splits * ATT_HEADS * 4 * 4);
}

__global__ void k_fill_zero(uint4* p, size_t n16) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

// Read-bandwidth probe: every 16-byte unit read once.  Workgroup w streams a
// contiguous share of the buffer in 4-KiB chunks (the waves taking chunks in
// turn, two in flight per wave), each chunk as four wave-wide 1-KiB
// non-temporal loads -- the access shape of the decode scoring stream; a tail
// shorter than a chunk is read by the first workgroup.  The words read are
// XOR-ed and the result stored only when it equals a value no caller supplies,
// so the loads are kept without a stream of atomics to one address.  The first
// wave also records the shader clock counter (s_memtime) and the 100 MHz
// constant clock (s_memrealtime) at its start and end.
__global__ __launch_bounds__(1024) void k_read_probe(const uint4* __restrict__ p, size_t n16, uint32_t* sink,
                                                    uint64_t* clocks) {
  uint64_t t0 = 0, r0 = 0;
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NWV = 16;
  const size_t nch = n16 / 256;  // whole 4-KiB chunks
  const size_t per = (nch + gridDim.x - 1) / gridDim.x;
  const size_t c_beg = (size_t)blockIdx.x * per;
  const size_t c_end = c_beg + per < nch ? c_beg + per : nch;
  uint32_t x = 0;
  const v4i* pv = reinterpret_cast<const v4i*>(p);
  auto ld = [&](size_t c, v4i (&v)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = c < c_end ? __builtin_nontemporal_load(pv + c * 256 + q * 64 + lane) : v4i{0, 0, 0, 0};
  };
  v4i a[4], b[4];
  size_t c = c_beg + wave;
  ld(c, a);
  ld(c + NWV, b);
  for (; c < c_end; c += 2 * NWV) {
#pragma unroll
    for (int q = 0; q < 4; ++q) x ^= (uint32_t)(a[q].x ^ a[q].y ^ a[q].z ^ a[q].w);
    ld(c + 2 * NWV, a);
    if (c + NWV >= c_end) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) x ^= (uint32_t)(b[q].x ^ b[q].y ^ b[q].z ^ b[q].w);
    ld(c + 3 * NWV, b);
  }
  if (blockIdx.x == 0)
    for (size_t i = nch * 256 + threadIdx.x; i < n16; i += blockDim.x) {
      const uint4 t = p[i];
      x ^= t.x ^ t.y ^ t.z ^ t.w;
    }
  if (x == 0x9E3779B9u) sink[0] = x;
  if (blockIdx.x == 0 && threadIdx.x == 0 && clocks) {
    clocks[0] = __builtin_amdgcn_s_memtime() - t0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

}  // namespace

isa_status launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  size_t n16 = bytes / 16;
  if (n16 == 0) return ISA_OK;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, (uint4*)p, n16);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

KernelTimer g_timer[3];

DevInfo device_info() {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static DevInfo cache[MAX_DEV];
  static bool known[MAX_DEV];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && known[dev]) return cache[dev];
  // an MI355X as a whole: the values used when a query fails
  DevInfo d{256, 8};
  int v = 0;
  if (dev >= 0 && hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
    d.n_cu = v;
  v = 0;
  if (dev >= 0 && hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0) d.n_xcd = v;
  if (d.n_xcd > d.n_cu) d.n_xcd = 1;
  if (dev >= 0) {
    cache[dev] = d;
    known[dev] = true;
  }
  return d;
}

// Argument checks of the decode-mode top-k beyond the batch description.
isa_status check_decode_topk(const int8_t* q, const int8_t* head_w, const int8_t* pooled, const isa_seqs* s,
                             const int32_t* scores_out, int32_t ld_scores) {
  if (!q || !head_w || !pooled || !aligned16(q) || !aligned16(head_w) || !aligned16(pooled))
    return ISA_ERR_INVALID_ARG;
  if (scores_out) {
    if (!aligned16(scores_out)) return ISA_ERR_INVALID_ARG;
    for (int b = 0; b < s->batch; ++b)
      if (groups_of(s->seq_lens_host[b]) > ld_scores) return ISA_ERR_INVALID_ARG;
  }
  return ISA_OK;
}

// Decode-mode scoring and selection on scratch laid out as `d` from `base`,
// device errors into `err`.
isa_status decode_topk(const int8_t* q, const int8_t* head_w, const int8_t* pooled, const isa_seqs* s, int32_t k,
                       int32_t* out_idx, int32_t* out_count, int32_t* scores_out, int32_t ld_scores,
                       const DecodeLayout& d, char* base, uint32_t* err, hipStream_t stream) {
  BatchArgs a;
  fill_batch(s, &a, k);
  a.tile_g = decode_tile_g(s);
  a.tile_skew = decode_tile_skew(a.tile_g);
  int t = 0;
  for (int b = 0; b < s->batch; ++b) {
    a.tile_start[b] = t;
    t += decode_tiles(s->seq_lens_host[b], k, a.tile_g);
  }
  a.tile_start[s->batch] = t;
  DecodeWs w{err, (uint2*)(base + d.tile_meta), (uint32_t*)(base + d.tile_pairs), (uint64_t*)(base + d.tile_list)};
  return launch_indexer_decode(a, q, head_w, pooled, s->block_table, w, out_idx, out_count, scores_out, ld_scores,
                               stream);
}

}  // namespace isa

// The top-k's scratch in a file-scope device array, for callers that cannot
// allocate (isa_indexer_topk_noalloc): isa_indexer_topk's workspace layout in
// ISA_NOALLOC_TOPK_BYTES bytes.  Each device holds its own copy, at its own
// address, looked up once per device with hipGetSymbolAddress; host code uses
// that address only, never the array's name.
static __device__ __align__(256) unsigned char scratch[ISA_NOALLOC_TOPK_BYTES];
static_assert(ISA_NOALLOC_TOPK_BYTES == isa::SCR0 + 384 * (8 + isa::PAIR_CAP * 4 + isa::TILE_CAP * 8),
              "the array holds the top-k layout of 384 work tiles");

using namespace isa;

extern "C" {

const char* isa_version(void) { return "isa 0.1 (gfx950)"; }

isa_status isa_set_kernel_timer(int32_t kernel, void* const* starts, void* const* stops, int32_t n) {
  if (kernel != ISA_TIMER_INDEXER_SCORE && kernel != ISA_TIMER_MLA_SPLIT) return ISA_ERR_INVALID_ARG;
  if (n < 0 || n > isa::TIMER_MAX || (n > 0 && (starts == nullptr || stops == nullptr))) return ISA_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (starts[i] == nullptr || stops[i] == nullptr) return ISA_ERR_INVALID_ARG;
  isa::KernelTimer& t = isa::g_timer[kernel];
  for (int i = 0; i < n; ++i) {
    t.start[i] = (hipEvent_t)starts[i];
    t.stop[i] = (hipEvent_t)stops[i];
  }
  t.next = 0;
  t.n = n;
  return ISA_OK;
}

const char* isa_status_string(isa_status st) {
  switch (st) {
    case ISA_OK: return "ok";
    case ISA_ERR_INVALID_ARG: return "invalid argument";
    case ISA_ERR_UNSUPPORTED: return "unsupported size";
    case ISA_ERR_WORKSPACE: return "workspace too small";
    case ISA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t isa_workspace_size(int op, const isa_seqs* s, int32_t rows, int32_t cols) {
  switch (op) {
    case ISA_OP_INDEXPOOL:
      return valid_seqs(s) ? pool_ws(s) : 0;
    case ISA_OP_INDEXER_TOPK:
      if (s == nullptr) return HDR;
      return valid_seqs(s) ? decode_layout(s, MAX_K).total : 0;
    case ISA_OP_SPARSE_MLA: {
      const int32_t layers = cols < 1 ? 1 : cols;
      return rows >= 1 && layers <= ISA_MAX_LAYERS ? mla_ws(rows, MAX_K, layers) : 0;
    }
    case ISA_OP_PREFILL_SCORES:
    case ISA_OP_APPEND_TOKEN:
    case ISA_OP_LATENT_FP8:
    case ISA_OP_KDA_STEP:
      return HDR;
  }
  return 0;
}

isa_status isa_read_probe(const void* buf, size_t bytes, uint32_t* sink, uint64_t* clocks, isa_stream_t stream) {
  if (!buf || !sink || !aligned16(buf) || ((uintptr_t)sink & 3) || ((uintptr_t)clocks & 7) || bytes == 0 ||
      (bytes & 15))
    return ISA_ERR_INVALID_ARG;
  // one 1024-thread workgroup per CU
  const unsigned grid = (unsigned)device_info().n_cu;
  hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(1024), 0, (hipStream_t)stream, (const uint4*)buf, bytes / 16, sink,
                     clocks);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

isa_status isa_workspace_init(void* ws, size_t ws_bytes, isa_stream_t stream) {
  if (!ws || !aligned16(ws) || ws_bytes < HDR || (ws_bytes & 15)) return ISA_ERR_INVALID_ARG;
  return launch_fill_zero(ws, ws_bytes, (hipStream_t)stream);
}

isa_status isa_device_error(void* ws, isa_stream_t stream, uint32_t* err_word, int clear) {
  if (!ws || !err_word) return ISA_ERR_INVALID_ARG;
  if (hipMemcpyAsync(err_word, ws, 4, hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess) return ISA_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return ISA_ERR_HIP;
  if (clear && *err_word) return launch_fill_zero(ws, 16, (hipStream_t)stream);
  return ISA_OK;
}

isa_status isa_indexpool(const uint16_t* keys, const float* w4, const isa_seqs* s, float* scales, int8_t* pooled,
                         uint32_t flags, void* ws, size_t ws_bytes, isa_stream_t stream) {
  if (!keys || !w4 || !scales || !pooled || !ws) return ISA_ERR_INVALID_ARG;
  if (!aligned16(keys) || !aligned16(pooled) || !aligned16(ws) || ((uintptr_t)scales & 3)) return ISA_ERR_INVALID_ARG;
  if (flags != ISA_SCALE_DYNAMIC && flags != ISA_SCALE_GIVEN) return ISA_ERR_INVALID_ARG;
  if (!valid_seqs(s)) return ISA_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (!(w4[i] == w4[i])) return ISA_ERR_INVALID_ARG;
  if (ws_bytes < pool_ws(s)) return ISA_ERR_WORKSPACE;
  BatchArgs a;
  fill_batch(s, &a, MAX_K);
  int t = 0;
  for (int b = 0; b < s->batch; ++b) {
    a.tile_start[b] = t;
    t += pool_tiles(s->seq_lens_host[b]);
  }
  a.tile_start[s->batch] = t;
  float* amax_part = reinterpret_cast<float*>((char*)ws + SCR0);
  return launch_indexpool(a, keys, w4, s->block_table, scales, pooled, flags == ISA_SCALE_DYNAMIC, amax_part,
                          (uint32_t*)ws, (hipStream_t)stream);
}

isa_status isa_indexer_topk(const int8_t* q, const int8_t* head_w, const int8_t* pooled, const isa_seqs* s,
                            const int32_t* scores_in, int32_t rows, int32_t ld_scores, int32_t k, int32_t* out_idx,
                            int32_t* out_count, int32_t* scores_out, void* ws, size_t ws_bytes,
                            isa_stream_t stream) {
  if (k < 1 || k > MAX_K || !out_idx || !out_count || !ws) return ISA_ERR_INVALID_ARG;
  if (!aligned16(out_idx) || !aligned16(out_count) || !aligned16(ws)) return ISA_ERR_INVALID_ARG;
  if (scores_in) {
    if (!aligned16(scores_in) || rows < 1 || ld_scores < 1) return ISA_ERR_INVALID_ARG;
    if (ws_bytes < HDR) return ISA_ERR_WORKSPACE;
    return launch_topk_rows(scores_in, rows, ld_scores, ld_scores, k, out_idx, out_count, (hipStream_t)stream);
  }
  if (!valid_seqs(s) || rows != s->batch) return ISA_ERR_INVALID_ARG;
  const isa_status st = check_decode_topk(q, head_w, pooled, s, scores_out, ld_scores);
  if (st != ISA_OK) return st;
  DecodeLayout d = decode_layout(s, k);
  if (ws_bytes < d.total) return ISA_ERR_WORKSPACE;
  return decode_topk(q, head_w, pooled, s, k, out_idx, out_count, scores_out, ld_scores, d, (char*)ws, (uint32_t*)ws,
                     (hipStream_t)stream);
}

isa_status isa_indexer_topk_noalloc(const int8_t* q, const int8_t* head_w, const int8_t* pooled, const isa_seqs* s,
                                    int32_t k, int32_t* out_idx, int32_t* out_count, int32_t* scores_out,
                                    int32_t ld_scores, uint32_t* err_word, isa_stream_t stream) {
  if (k < 1 || k > MAX_K || !out_idx || !out_count || !err_word) return ISA_ERR_INVALID_ARG;
  if (!aligned16(out_idx) || !aligned16(out_count) || ((uintptr_t)err_word & 3)) return ISA_ERR_INVALID_ARG;
  if (!valid_seqs(s)) return ISA_ERR_INVALID_ARG;
  const isa_status st = check_decode_topk(q, head_w, pooled, s, scores_out, ld_scores);
  if (st != ISA_OK) return st;
  DecodeLayout d = decode_layout(s, k);
  if (d.total > ISA_NOALLOC_TOPK_BYTES) return ISA_ERR_UNSUPPORTED;
  // the array's device address, once per device, with that device current
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static char* addr[MAX_DEV];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return ISA_ERR_HIP;
  char* base;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return ISA_ERR_HIP;
      addr[dev] = (char*)ptr;
    }
    base = addr[dev];
  }
  return decode_topk(q, head_w, pooled, s, k, out_idx, out_count, scores_out, ld_scores, d, base, err_word,
                     (hipStream_t)stream);
}


static isa_status sparse_mla(int32_t n_layers, const uint16_t* const* q, const void* const* latent,
                             const float* const* lat_scale, const isa_seqs* s, const int32_t* row_seq,
                             const int32_t* row_pos, int32_t rows, const int32_t* idx, const int32_t* count,
                             int32_t k, float sm_scale, float* const* out, float* const* lse, void* ws,
                             size_t ws_bytes, isa_stream_t stream) {
  if (n_layers < 1 || n_layers > ISA_MAX_LAYERS || !q || !latent || !out) return ISA_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l) {
    if (!q[l] || !latent[l] || !out[l] || (lse && !lse[l]) || (lat_scale && !lat_scale[l]))
      return ISA_ERR_INVALID_ARG;
    if (!aligned16(q[l]) || !aligned16(latent[l]) || !aligned16(out[l]) || (lse && !aligned16(lse[l])) ||
        (lat_scale && !aligned16(lat_scale[l])))
      return ISA_ERR_INVALID_ARG;
  }
  if (!idx || !count || !ws) return ISA_ERR_INVALID_ARG;
  if (!aligned16(idx) || !aligned16(count) || !aligned16(ws) || (row_seq && !aligned16(row_seq)) ||
      (row_pos && !aligned16(row_pos)))
    return ISA_ERR_INVALID_ARG;
  if (k < 1 || k > MAX_K || rows < 1 || !(sm_scale > 0.f) || sm_scale != sm_scale) return ISA_ERR_INVALID_ARG;
  if (!valid_seqs(s)) return ISA_ERR_INVALID_ARG;
  if (!row_seq && rows > s->batch) return ISA_ERR_INVALID_ARG;
  MlaPlan p = plan_mla(rows, k, n_layers);
  if ((long long)rows * p.splits * n_layers * ATT_HEADS > 0x7FFFFFFF) return ISA_ERR_UNSUPPORTED;
  if (ws_bytes < mla_ws(rows, k, n_layers)) return ISA_ERR_WORKSPACE;
  BatchArgs a;
  fill_batch(s, &a, k);
  char* base = (char*)ws;
  MlaWs w{(uint32_t*)base, base + SCR0,
          (float*)(base + SCR0 + up256((size_t)n_layers * rows * p.splits * ATT_HEADS * LAT_DIM * 4))};
  return launch_sparse_mla(a, p, n_layers, q, latent, lat_scale, s->block_table, row_seq, row_pos, idx, count, k,
                           sm_scale, out, lse, w, (hipStream_t)stream);
}

isa_status isa_sparse_mla_decode(const uint16_t* q, const uint16_t* latent, const isa_seqs* s,
                                 const int32_t* row_seq, const int32_t* row_pos, int32_t rows, const int32_t* idx,
                                 const int32_t* count, int32_t k, float sm_scale, float* out, float* lse, void* ws,
                                 size_t ws_bytes, isa_stream_t stream) {
  if (!q || !latent || !out) return ISA_ERR_INVALID_ARG;
  const void* lat = latent;
  return sparse_mla(1, &q, &lat, nullptr, s, row_seq, row_pos, rows, idx, count, k, sm_scale, &out,
                    lse ? &lse : nullptr, ws, ws_bytes, stream);
}

isa_status isa_sparse_mla_decode_fp8(const uint16_t* q, const uint8_t* codes, const float* row_scales,
                                     const isa_seqs* s, const int32_t* row_seq, const int32_t* row_pos, int32_t rows,
                                     const int32_t* idx, const int32_t* count, int32_t k, float sm_scale, float* out,
                                     float* lse, void* ws, size_t ws_bytes, isa_stream_t stream) {
  if (!q || !codes || !row_scales || !out) return ISA_ERR_INVALID_ARG;
  const void* lat = codes;
  return sparse_mla(1, &q, &lat, &row_scales, s, row_seq, row_pos, rows, idx, count, k, sm_scale, &out,
                    lse ? &lse : nullptr, ws, ws_bytes, stream);
}

isa_status isa_sparse_mla_decode_shared(int32_t n_layers, const uint16_t* const* q, const uint16_t* const* latent,
                                        const isa_seqs* s, const int32_t* row_seq, const int32_t* row_pos,
                                        int32_t rows, const int32_t* idx, const int32_t* count, int32_t k,
                                        float sm_scale, float* const* out, float* const* lse, void* ws,
                                        size_t ws_bytes, isa_stream_t stream) {
  if (!latent || n_layers < 1 || n_layers > ISA_MAX_LAYERS) return ISA_ERR_INVALID_ARG;
  const void* lat[ISA_MAX_LAYERS];
  for (int l = 0; l < n_layers; ++l) lat[l] = latent[l];
  return sparse_mla(n_layers, q, lat, nullptr, s, row_seq, row_pos, rows, idx, count, k, sm_scale, out, lse, ws,
                    ws_bytes, stream);
}

isa_status isa_append_token(const uint16_t* key_new, const uint16_t* latent_new, const float* w4, const isa_seqs* s,
                            const float* scales, uint16_t* keys, uint16_t* latent, int8_t* pooled, void* ws,
                            size_t ws_bytes, isa_stream_t stream) {
  if (!key_new || !w4 || !scales || !keys || !pooled || !ws) return ISA_ERR_INVALID_ARG;
  if ((latent_new == nullptr) != (latent == nullptr)) return ISA_ERR_INVALID_ARG;
  if (!aligned16(key_new) || !aligned16(keys) || !aligned16(pooled) || !aligned16(ws) || ((uintptr_t)scales & 3) ||
      (latent_new && (!aligned16(latent_new) || !aligned16(latent))))
    return ISA_ERR_INVALID_ARG;
  if (!valid_seqs(s)) return ISA_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (!(w4[i] == w4[i])) return ISA_ERR_INVALID_ARG;
  if (ws_bytes < HDR) return ISA_ERR_WORKSPACE;
  BatchArgs a;
  fill_batch(s, &a, MAX_K);
  return launch_append(a, key_new, latent_new, w4, s->block_table, scales, keys, latent, pooled, (uint32_t*)ws,
                       (hipStream_t)stream);
}

isa_status isa_latent_to_fp8(const uint16_t* latent, const isa_seqs* s, uint8_t* codes, float* row_scales, void* ws,
                             size_t ws_bytes, isa_stream_t stream) {
  if (!latent || !codes || !row_scales || !ws) return ISA_ERR_INVALID_ARG;
  if (!aligned16(latent) || !aligned16(codes) || !aligned16(row_scales) || !aligned16(ws)) return ISA_ERR_INVALID_ARG;
  if (!valid_seqs(s)) return ISA_ERR_INVALID_ARG;
  if (ws_bytes < HDR) return ISA_ERR_WORKSPACE;
  BatchArgs a;
  fill_batch(s, &a, MAX_K);
  int t = 0;
  for (int b = 0; b < s->batch; ++b) {
    a.tile_start[b] = t;
    t += (s->seq_lens_host[b] + PAGE_TOK - 1) / PAGE_TOK;  // one workgroup per page
  }
  a.tile_start[s->batch] = t;
  return launch_latent_fp8(a, latent, s->block_table, codes, row_scales, (uint32_t*)ws, (hipStream_t)stream);
}

isa_status isa_kda_decode_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                               const float* beta, uint16_t* state, float* out, int32_t n, void* ws, size_t ws_bytes,
                               isa_stream_t stream) {
  if (!q || !k || !v || !alpha || !beta || !state || !out || !ws) return ISA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(alpha) || !aligned16(beta) ||
      !aligned16(state) || !aligned16(out) || !aligned16(ws))
    return ISA_ERR_INVALID_ARG;
  if (n < 1) return ISA_ERR_INVALID_ARG;
  if (ws_bytes < HDR) return ISA_ERR_WORKSPACE;
  return launch_kda_step(q, k, v, alpha, beta, state, out, n, (uint32_t*)ws, (hipStream_t)stream);
}

isa_status isa_indexer_prefill_scores(const int8_t* q, const int8_t* head_w, const int32_t* q_pos, int32_t Q,
                                      const int8_t* pooled, const isa_seqs* s, int32_t* scores, int32_t ld_scores,
                                      void* ws, size_t ws_bytes, isa_stream_t stream) {
  if (!q || !head_w || !q_pos || !pooled || !scores || !ws) return ISA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(head_w) || !aligned16(q_pos) || !aligned16(pooled) || !aligned16(scores) ||
      !aligned16(ws))
    return ISA_ERR_INVALID_ARG;
  if (Q < 1 || !valid_seqs(s) || s->batch != 1) return ISA_ERR_INVALID_ARG;
  if (groups_of(s->seq_lens_host[0]) > ld_scores) return ISA_ERR_INVALID_ARG;
  if (ws_bytes < HDR) return ISA_ERR_WORKSPACE;
  BatchArgs a;
  fill_batch(s, &a, MAX_K);
  return launch_prefill_scores(a, q, head_w, q_pos, Q, pooled, s->block_table, scores, ld_scores, (uint32_t*)ws,
                               (hipStream_t)stream);
}

}  // extern "C"
