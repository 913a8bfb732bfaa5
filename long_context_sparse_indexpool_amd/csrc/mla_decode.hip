// mla_decode.hip -- sparse NoPE MLA softmax attention over the selected latent
// rows, gfx950.
//
// Method (pages cited by title): "GLM-5.3-Flash: 하이브리드 희소·선형 어텐션과
// IndexPool·EPD로 1M 컨텍스트를 오픈 소스로 서빙하는 방법" (llm-wiki.hwlabs.dev),
// section "희소 어텐션: 인덱서로 필요한 토큰만": softmax attention over only the
// positions the indexer selected.  "GLM-5.3 Sparse Attention은 연산량을 줄이지만 HBM
// 수요는 지속된다" (remio.ai), section "GLM-5.3 Sparse Attention이 실제로 바꾸는 것":
// MLA caches one compressed latent per token and attention reads only the
// selected rows.  "GLM-5.3-Flash vs Qwen3.8-Flash-Next" (alltoptrend), section
// "의견이 갈리는 지점 — 위치 인코딩": qk_rope_head_dim = 0, so no rotary part.  The
// absorbed form is used: keys = values = the 512-d latent row.
//
// Design.  A workgroup is (query row, token split) with eight waves: wave w owns
// heads 16(w%4)..+15 and latent channels 256(w/4)..+255, so each wave's output
// accumulator is 16 heads x 256 channels (64 registers per lane).  The split's
// selected groups are first turned into a table of physical latent rows (one
// block-table lookup per group).  Then, per tile of 16 tokens:
//  * Partial scores S^T = C Q^T over the wave's 256 channels with
//    v_mfma_f32_16x16x32_bf16: tokens are M, the wave's 16 heads are N.  Each
//    lane loads 16 contiguous bytes of a latent row per K step straight from
//    HBM into a ring of register slots; a slot is refilled with the next tile's
//    K step as soon as it is consumed, so a whole tile of loads is in flight.
//    The two waves sharing a head block add their halves through LDS (both
//    then hold identical scores and make identical softmax decisions).
//  * Each wave also converts one eighth of the tile's channels to fp16 (exact
//    for bf16 values inside the fp16 range) and stores them transposed in LDS
//    (V^T).  Computing S^T leaves every lane with four probabilities of one
//    head in exactly the A-operand layout the P.V product needs.
//  * Softmax in fp32, base 2.  The exponent reference of a head moves only when
//    its running max exceeds it by more than 8 (so p <= 256 in fp16), which
//    makes the rescale of the output accumulator rare.
//  * O += P V with v_mfma_f32_16x16x16f16: heads are M, 16 channels per N
//    block, the 16 tokens are K; V^T comes from LDS with one 8-byte read.
// With one split the workgroup normalises and writes the output; otherwise it
// writes its unnormalised partial (O, reference, sum) and k_mla_combine merges
// the splits by log-sum-exp weights.
#include "isa_launch.hpp"

namespace isa {

constexpr int MLA_THREADS = 512;  // 8 waves: 4 head blocks x 2 channel halves
constexpr int HALF_DIM = LAT_DIM / 2;
constexpr int KSTEPS = HALF_DIM / 32;  // K steps of the score product per wave
constexpr int NBLK = HALF_DIM / 16;    // 16-channel blocks of the output per wave
constexpr float RESCALE_LOG2 = 8.f;

// token slot inside the 32-token K block, in the order the S^T accumulators
// hand the probabilities to the P.V operand
__device__ __forceinline__ int kperm(int t) { return 8 * ((t & 15) >> 2) + (t & 3) + 4 * (t >> 4); }
constexpr int TILE_TOK = 32;
constexpr int TILE_GRP = TILE_TOK / GROUP;
constexpr int VT_STRIDE = 40;  // halves per V^T row (32 tokens + 8 pad, 80 B)
constexpr int MAX_GPS = MAX_K; // groups per split held in LDS
constexpr int MAX_SPLITS = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Two bf16 values (low half first) to two fp16 values.  Exact for values in
// the fp16 normal range, which the latent rows are required to stay in; the
// conversion truncates, which for these values is the same as rounding.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
  return __builtin_bit_cast(uint32_t, h);
}
// low (high) halves of a and b, a's in the low half of the result
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }
// 4x4 transpose inside each quad of lanes: lane i holds v = M[i][0..3] on
// entry and M[0..3][i] on exit.  Two exchange rounds (lane bit 0 with element
// bit 0, then bit 1 with bit 1), each a DPP quad permutation plus selects.
__device__ __forceinline__ void quad_transpose(uint32_t (&v)[4], int i) {
  const bool b0 = i & 1, b1 = i & 2;
#pragma unroll
  for (int p = 0; p < 4; p += 2) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(b0 ? v[p] : v[p + 1]), 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    v[p] = b0 ? r : v[p];
    v[p + 1] = b0 ? v[p + 1] : r;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)(b1 ? v[p] : v[p + 2]), 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    v[p] = b1 ? r : v[p];
    v[p + 2] = b1 ? v[p + 2] : r;
  }
}

struct MlaPtrs {
  const uint16_t* q;
  const uint16_t* latent;
  const int32_t* bt;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const int32_t* idx;
  const int32_t* count;
  float* out;
  float* lse;
  float* o_part;
  float* ml_part;
  uint32_t* err;
  int32_t k;
  float c2;  // sm_scale * log2(e)
  int32_t splits;
  int32_t gps;  // groups per split
};

__global__ __launch_bounds__(MLA_THREADS) void k_mla_split(const BatchArgs a, const MlaPtrs P) {
  __shared__ _Float16 vt[2][LAT_DIM * VT_STRIDE];  // 2 x 40 KiB: V^T of a 32-token tile, double-buffered
  __shared__ v4f sx[2][2][MLA_THREADS];            // 2 x 16 KiB: partial scores exchanged between wave pairs
  __shared__ uint32_t trow[MAX_GPS * GROUP];    // latent row of each token slot, or ~0 if not visible

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hb = wave & 3, half = wave >> 2;  // heads 16hb.., channels 256half..
  const int r = blockIdx.x / P.splits;
  const int split = blockIdx.x % P.splits;
  const int lq = lane & 15, lg = lane >> 4;  // column / row-group of the 16x16 layouts

  // row description, read by every thread (no barrier); the split's group ids
  // are fetched in the same round, before the count is known
  int seq = P.row_seq ? P.row_seq[r] : r;
  const bool seq_ok = seq >= 0 && seq < a.batch;
  if (!seq_ok) seq = 0;
  const int L = seq_ok ? a.lens[seq] : 0;
  const int pos = seq_ok ? (P.row_pos ? P.row_pos[r] : L - 1) : -1;
  int cnt = P.count[r];
  const int jbeg0 = split * P.gps;
  int gid[MAX_GPS / MLA_THREADS + 1];
#pragma unroll
  for (int e = 0; e < MAX_GPS / MLA_THREADS + 1; ++e) {
    const int j = tid + e * MLA_THREADS;
    gid[e] = (j < P.gps && jbeg0 + j < P.k) ? P.idx[(size_t)r * P.k + jbeg0 + j] : -1;
  }
  if (!seq_ok || pos < 0 || pos >= L || cnt < 0 || cnt > P.k) {
    if (tid == 0) report(P.err, ISA_DERR_ROW_RANGE);
    cnt = 0;
  }
  const int G = (L + GROUP - 1) / GROUP;
  const int jbeg = min(cnt, jbeg0);
  const int jend = min(cnt, jbeg + P.gps);
  const int ng = jend - jbeg;
  // token table of the split: one block-table lookup per selected group
#pragma unroll
  for (int e = 0; e < MAX_GPS / MLA_THREADS + 1; ++e) {
    const int j = tid + e * MLA_THREADS;
    if (j >= ng) continue;
    const int g = gid[e];
    int pg = -1;
    if (g < 0 || g >= G) report(P.err, ISA_DERR_ROW_RANGE);
    else pg = phys_page(P.bt, a.max_pages, a.num_pages, seq, (g * GROUP) / PAGE_TOK, P.err);
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      int tok = g * GROUP + i;
      bool vis = pg >= 0 && tok < L && tok <= pos;
      trow[j * GROUP + i] = vis ? (uint32_t)pg * PAGE_TOK + (uint32_t)(tok % PAGE_TOK) : 0xFFFFFFFFu;
    }
  }

  // query operand (B = Q^T): lane -> head 16hb + lq, channels 256half + 32c + 8lg .. +7
  v8bf qop[KSTEPS];
  {
    const uint16_t* qp = P.q + ((size_t)r * ATT_HEADS + hb * 16 + lq) * LAT_DIM + half * HALF_DIM + lg * 8;
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      v4i v = *reinterpret_cast<const v4i*>(qp + c * 32);
      qop[c] = __builtin_bit_cast(v8bf, v);
    }
  }
  v4f o[NBLK];
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb) o[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;  // exponent reference (log2 units) and partial sum of the head
  __syncthreads();

  const int nslot = ng * GROUP;
  const int ntile = (nslot + TILE_TOK - 1) / TILE_TOK;
  // QK operand of a tile: for each 16-token block bk, token row bk*16 + lq,
  // channels 256half + 32c + 8lg .. +7.  Loads are unconditional (an invisible
  // token reads row 0 of the pool and is zeroed by a mask), so no branch
  // separates a load from its use and the compiler waits for exactly the slot
  // it consumes; each slot is refilled with the next tile's K step as soon as
  // it has been consumed, so a whole tile of loads stays in flight.
  auto row_of = [&](int tile, int bk, int& mask) -> const v4i* {
    const int slot = tile * TILE_TOK + bk * 16 + lq;
    const uint32_t t = trow[min(slot, MAX_GPS * GROUP - 1)];  // always in range; masked below
    const bool vis = tile < ntile && slot < nslot && t != 0xFFFFFFFFu;
    mask = vis ? -1 : 0;
    const uint32_t row = vis ? t : 0u;
    return reinterpret_cast<const v4i*>(P.latent + (size_t)row * LAT_DIM + half * HALF_DIM + lg * 8);
  };
  // The first tile is issued in the loop's own order (K step by K step, both
  // token blocks), pinned by scheduling barriers: the wait counter at the loop
  // head merges this entry with the back edge, so any other order here would
  // turn the per-slot waits into a wait for every load.
  v4i buf[2][KSTEPS];
  int bmask[2];
  {
    const v4i* src0 = row_of(0, 0, bmask[0]);
    const v4i* src1 = row_of(0, 1, bmask[1]);
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      buf[0][c] = src0[c * 4];
      buf[1][c] = src1[c * 4];
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (int tile = 0; tile < ntile; ++tile) {
    const int vb = tile & 1;  // V^T / exchange buffer of this tile
    _Float16* vtb = vt[vb];
    // visibility of the tile's tokens: bit t of vis[bk] <-> token bk*16 + t
    const uint64_t vis0 = __ballot(bmask[0] != 0), vis1 = __ballot(bmask[1] != 0);
    int nmask[2];
    const v4i* nsrc0 = row_of(tile + 1, 0, nmask[0]);
    const v4i* nsrc1 = row_of(tile + 1, 1, nmask[1]);
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      const v4i r0 = buf[0][c] & bmask[0], r1 = buf[1][c] & bmask[1];
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, r0), qop[c], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, r1), qop[c], s1, 0, 0, 0);
      if ((c >> 1) == hb) {  // this wave's eighth of V^T: channels 256half + 32c + 8lg .. +7
        // Lane (m = lq/4, i = lq%4) holds tokens at slots 8m+i (block 0) and
        // 8m+4+i (block 1).  A 4x4 transpose of channel pairs inside the quad
        // gives lane i channels 2i, 2i+1 of all eight slots 8m..8m+7, which it
        // stores as two 16-byte rows of V^T.
        uint32_t x[4], y[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          x[p] = bf16x2_to_f16x2((uint32_t)r0[p]);
          y[p] = bf16x2_to_f16x2((uint32_t)r1[p]);
        }
        const int qi = lq & 3;
        quad_transpose(x, qi);
        quad_transpose(y, qi);
        const int d = half * HALF_DIM + c * 32 + lg * 8 + 2 * qi;
        const int slot = 8 * (lq >> 2);
        const v4i lo = {(int)pack_lo(x[0], x[1]), (int)pack_lo(x[2], x[3]), (int)pack_lo(y[0], y[1]),
                        (int)pack_lo(y[2], y[3])};
        const v4i hi = {(int)pack_hi(x[0], x[1]), (int)pack_hi(x[2], x[3]), (int)pack_hi(y[0], y[1]),
                        (int)pack_hi(y[2], y[3])};
        *reinterpret_cast<v4i*>(&vtb[d * VT_STRIDE + slot]) = lo;
        *reinterpret_cast<v4i*>(&vtb[(d + 1) * VT_STRIDE + slot]) = hi;
      }
      buf[0][c] = nsrc0[c * 4];
      buf[1][c] = nsrc1[c * 4];
    }
    bmask[0] = nmask[0];
    bmask[1] = nmask[1];
    sx[vb][0][tid] = s0;
    sx[vb][1][tid] = s1;
    lds_barrier();  // V^T and partial scores of this tile complete (double-buffered: one barrier per tile)
    const v4f o0 = sx[vb][0][tid ^ (4 * 64)], o1 = sx[vb][1][tid ^ (4 * 64)];  // the other channel half
    // the accumulators hold head lq of tokens 4lg + i (block 0) and 16 + 4lg + i (block 1)
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (vis0 >> (4 * lg + i)) & 1 ? (s0[i] + o0[i]) * P.c2 : -INFINITY;
      x[4 + i] = (vis1 >> (4 * lg + i)) & 1 ? (s1[i] + o1[i]) * P.c2 : -INFINITY;
    }
    float mt = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, x[i]);
    // move the exponent reference only when some head's scores got 2^8 above it
    // (p then stays <= 256); the max over the four lanes of a head is needed
    // only then.  Both waves of a head block see identical scores.
    if (__any(mt > m_ref + RESCALE_LOG2)) {
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_ref - m_new);
      l_run *= alpha;
      m_ref = m_new;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * lg + i, 64);
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nb][i] *= al[i];
    }
    v8h pop;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = m_ref == -INFINITY ? 0.f : exp2f(x[i] - m_ref);
      ps += p;
      pop[i] = (_Float16)p;
    }
    l_run += ps;
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) {
      const v4i vv = *reinterpret_cast<const v4i*>(&vtb[(half * HALF_DIM + nb * 16 + lq) * VT_STRIDE + lg * 8]);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, __builtin_bit_cast(v8h, vv), o[nb], 0, 0, 0);
    }
  }

  // per-head sum over the four lanes holding the head
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int h0 = hb * 16;
  const int d_base = half * HALF_DIM;
  if (P.splits == 1) {
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float li = __shfl(l_tot, 4 * lg + i, 64);
      inv[i] = li > 0.f ? 1.f / li : 0.f;
    }
    float* orow = P.out + (size_t)r * ATT_HEADS * LAT_DIM;
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        orow[(size_t)(h0 + 4 * lg + i) * LAT_DIM + d_base + nb * 16 + lq] = o[nb][i] * inv[i];
    if (P.lse && half == 0 && lane < 16)
      P.lse[(size_t)r * ATT_HEADS + h0 + lq] = l_tot > 0.f ? m_ref * LN2 + logf(l_tot) : -INFINITY;
  } else {
    float* op = P.o_part + ((size_t)r * P.splits + split) * ATT_HEADS * LAT_DIM;
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) op[(size_t)(h0 + 4 * lg + i) * LAT_DIM + d_base + nb * 16 + lq] = o[nb][i];
    if (half == 0 && lane < 16) {
      float* mp = P.ml_part + (((size_t)r * P.splits + split) * ATT_HEADS + h0 + lq) * 2;
      mp[0] = l_tot > 0.f ? m_ref : -INFINITY;
      mp[1] = l_tot;
    }
  }
}

// Merge the splits of one (row, head): weights 2^(m_s - M), then a weighted
// sum of the partial outputs (128 threads x 4 channels, loads unrolled).
__global__ __launch_bounds__(128) void k_mla_combine(const MlaPtrs P) {
  __shared__ float wsh[MAX_SPLITS];
  __shared__ float stat[2];
  const int r = blockIdx.x / ATT_HEADS, h = blockIdx.x % ATT_HEADS;
  const int S = P.splits;
  const float* ml = P.ml_part + ((size_t)r * S * ATT_HEADS + h) * 2;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float m = lane < S ? ml[(size_t)lane * ATT_HEADS * 2] : -INFINITY;
    float l = lane < S ? ml[(size_t)lane * ATT_HEADS * 2 + 1] : 0.f;
    float M = m;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float w = (M == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - M);
    float ws = w * l;
    for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o, 64);
    if (lane < S) wsh[lane] = ws > 0.f ? w / ws : 0.f;
    if (lane == 0) {
      stat[0] = M;
      stat[1] = ws;
    }
  }
  __syncthreads();
  const float* op = P.o_part + ((size_t)r * S * ATT_HEADS + h) * LAT_DIM + threadIdx.x * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    float f = wsh[s];
    float4 v = *reinterpret_cast<const float4*>(op + (size_t)s * ATT_HEADS * LAT_DIM);
    acc.x = fmaf(f, v.x, acc.x);
    acc.y = fmaf(f, v.y, acc.y);
    acc.z = fmaf(f, v.z, acc.z);
    acc.w = fmaf(f, v.w, acc.w);
  }
  *reinterpret_cast<float4*>(P.out + ((size_t)r * ATT_HEADS + h) * LAT_DIM + threadIdx.x * 4) = acc;
  if (P.lse && threadIdx.x == 0)
    P.lse[(size_t)r * ATT_HEADS + h] = stat[1] > 0.f ? stat[0] * LN2 + logf(stat[1]) : -INFINITY;
}

MlaPlan plan_mla(int32_t rows, int32_t k) {
  // about 256 workgroups in flight, at least 16 groups (64 tokens) per split
  MlaPlan p;
  p.rows = rows;
  int s = (256 + rows - 1) / rows;
  int smax = (k + 15) / 16;
  if (s > smax) s = smax;
  if (s > MAX_SPLITS) s = MAX_SPLITS;
  if (s < 1) s = 1;
  p.splits = s;
  p.groups_per_split = (k + s - 1) / s;
  return p;
}

isa_status launch_sparse_mla(const BatchArgs& a, const MlaPlan& p, const uint16_t* q, const uint16_t* latent,
                             const int32_t* bt, const int32_t* row_seq, const int32_t* row_pos,
                             const int32_t* idx, const int32_t* count, int32_t k, float sm_scale, float* out,
                             float* lse, const MlaWs& w, hipStream_t stream) {
  MlaPtrs P{q, latent, bt, row_seq, row_pos, idx, count, out, lse, w.o_part, w.ml_part, w.err, k,
            sm_scale * LOG2E, p.splits, p.groups_per_split};
  timer_begin(ISA_TIMER_MLA_SPLIT, stream);
  hipLaunchKernelGGL(k_mla_split, dim3(p.rows * p.splits), dim3(MLA_THREADS), 0, stream, a, P);
  if (hipGetLastError() != hipSuccess) return ISA_ERR_HIP;
  timer_end(ISA_TIMER_MLA_SPLIT, stream);
  if (p.splits > 1) {
    hipLaunchKernelGGL(k_mla_combine, dim3(p.rows * ATT_HEADS), dim3(128), 0, stream, P);
    if (hipGetLastError() != hipSuccess) return ISA_ERR_HIP;
  }
  return ISA_OK;
}

}  // namespace isa
