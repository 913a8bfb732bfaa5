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
// Design.  A workgroup is (query row, token split) with four waves; wave w owns
// heads 16w..16w+15 and the whole split, in tiles of 32 tokens (8 groups).
// Per tile:
//  * Scores as S^T = C Q^T with v_mfma_f32_16x16x32_bf16: tokens are M, the
//    wave's 16 heads are N, the 512 channels the K loop.  Each lane loads 16
//    contiguous bytes of a latent row per K step straight from HBM (the rows
//    of a group are contiguous in a page); the query operand stays in
//    registers.  Computing S^T makes each lane hold 8 probabilities of one
//    head, which is exactly the A operand layout the PV product needs.
//  * While loading, wave w converts channels 128w..128w+127 of the tile to fp16
//    (exact for bf16 values in fp16 range) and stores them transposed into LDS
//    (V^T, rows padded to 80 B against bank conflicts), in the token order the
//    probability operand uses.
//  * Online softmax in fp32 (base 2; the running max per head is reduced across
//    the four lanes holding it; the output rescale is skipped when no head of
//    the wave raised its max).
//  * O += P V with v_mfma_f32_16x16x32_f16: heads as M, 16 channels per N block,
//    the 32 tokens as K; V^T comes from LDS with one 16-byte read per MFMA.
// With one split the workgroup normalises and writes the output; otherwise it
// writes its unnormalised partial (O, max, sum) and a combine kernel merges
// the splits by log-sum-exp weights.
#include "isa_launch.hpp"

namespace isa {

constexpr int MLA_THREADS = 256;
constexpr int TILE_TOK = 32;
constexpr int TILE_GRP = TILE_TOK / GROUP;
constexpr int VT_STRIDE = 40;  // halves per V^T row (32 tokens + 8 pad)
constexpr int MAX_GPS = MAX_K; // groups per split held in LDS
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

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

// token slot inside the 32-token K block, as laid out by the S^T accumulators
__device__ __forceinline__ int kperm(int t) { return 8 * ((t & 15) >> 2) + (t & 3) + 4 * (t >> 4); }

__global__ __launch_bounds__(MLA_THREADS) void k_mla_split(const BatchArgs a, const MlaPtrs P) {
  __shared__ _Float16 vt[LAT_DIM * VT_STRIDE];  // 40 KiB
  __shared__ int32_t sidx[MAX_GPS];
  __shared__ int32_t rowinfo[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x / P.splits;
  const int split = blockIdx.x % P.splits;
  const int lq = lane & 15, lg = lane >> 4;  // column / row-group of the 16x16 layouts

  if (tid == 0) {
    int seq = P.row_seq ? P.row_seq[r] : r;
    int ok = seq >= 0 && seq < a.batch;
    int L = ok ? a.lens[seq] : 0;
    int pos = ok ? (P.row_pos ? P.row_pos[r] : L - 1) : -1;
    int cnt = P.count[r];
    if (!ok || pos < 0 || pos >= L || cnt < 0 || cnt > P.k) {
      report(P.err, ISA_DERR_ROW_RANGE);
      cnt = 0;
    }
    rowinfo[0] = ok ? seq : 0;
    rowinfo[1] = L;
    rowinfo[2] = pos;
    rowinfo[3] = cnt;
  }
  __syncthreads();
  const int seq = rowinfo[0], L = rowinfo[1], pos = rowinfo[2], cnt = rowinfo[3];
  const int G = (L + GROUP - 1) / GROUP;
  const int jbeg = min(cnt, split * P.gps);
  const int jend = min(cnt, jbeg + P.gps);
  const int ng = jend - jbeg;
  for (int j = tid; j < ng; j += MLA_THREADS) {
    int g = P.idx[(size_t)r * P.k + jbeg + j];
    if (g < 0 || g >= G) {
      report(P.err, ISA_DERR_ROW_RANGE);
      g = -1;
    }
    sidx[j] = g;
  }

  // query operand (B = Q^T): lane -> head 16w + lq, channels 32c + 8lg .. +7
  v8bf qop[16];
  {
    const uint16_t* qp = P.q + ((size_t)r * ATT_HEADS + wave * 16 + lq) * LAT_DIM + lg * 8;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      v4i v = *reinterpret_cast<const v4i*>(qp + c * 32);
      qop[c] = __builtin_bit_cast(v8bf, v);
    }
  }
  v4f o[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) o[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();

  const int ntile = (ng + TILE_GRP - 1) / TILE_GRP;
  for (int tile = 0; tile < ntile; ++tile) {
    const int jt = tile * TILE_GRP;
    // rows this lane loads: tokens t = lq (+16): group slot t/4, token 4g + t%4
    const uint16_t* src[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      int t = bk * 16 + lq;
      int js = jt + (t >> 2);
      src[bk] = nullptr;
      if (js < ng) {
        int g = sidx[js];
        int tok = 4 * g + (t & 3);
        if (g >= 0 && tok < L && tok <= pos) {
          int pg = phys_page(P.bt, a.max_pages, a.num_pages, seq, tok / PAGE_TOK, P.err);
          if (pg >= 0) src[bk] = P.latent + ((size_t)pg * PAGE_TOK + (tok % PAGE_TOK)) * LAT_DIM + lg * 8;
        }
      }
    }
    // S^T = C Q^T over 16 K steps of 32 channels
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      v4i r0 = src[0] ? *reinterpret_cast<const v4i*>(src[0] + c * 32) : v4i{0, 0, 0, 0};
      v4i r1 = src[1] ? *reinterpret_cast<const v4i*>(src[1] + c * 32) : v4i{0, 0, 0, 0};
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, r0), qop[c], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, r1), qop[c], s1, 0, 0, 0);
      if ((c >> 2) == wave) {  // this wave's quarter of V^T
        const int d0 = c * 32 + lg * 8;
        const int k0 = kperm(lq), k1 = kperm(16 + lq);
        const uint32_t w0[4] = {(uint32_t)r0.x, (uint32_t)r0.y, (uint32_t)r0.z, (uint32_t)r0.w};
        const uint32_t w1[4] = {(uint32_t)r1.x, (uint32_t)r1.y, (uint32_t)r1.z, (uint32_t)r1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vt[(d0 + 2 * i) * VT_STRIDE + k0] = (_Float16)__uint_as_float(w0[i] << 16);
          vt[(d0 + 2 * i + 1) * VT_STRIDE + k0] = (_Float16)__uint_as_float(w0[i] & 0xFFFF0000u);
          vt[(d0 + 2 * i) * VT_STRIDE + k1] = (_Float16)__uint_as_float(w1[i] << 16);
          vt[(d0 + 2 * i + 1) * VT_STRIDE + k1] = (_Float16)__uint_as_float(w1[i] & 0xFFFF0000u);
        }
      }
    }
    // visibility of the accumulator tokens: t = 16bk + 4lg + i -> group slot 4bk + lg
    float x[8];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      int js = jt + 4 * bk + lg;
      int g = js < ng ? sidx[js] : -1;
      v4f s = bk ? s1 : s0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int tok = 4 * g + i;
        bool vis = g >= 0 && tok < L && tok <= pos;
        x[bk * 4 + i] = vis ? s[i] * P.c2 : -INFINITY;
      }
    }
    float mt = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, x[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    float alpha = 1.f;
    v8h pop;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pop[i] = (_Float16)0.f;
    } else {
      alpha = exp2f(m_run - m_new);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p = exp2f(x[i] - m_new);
        ps += p;
        pop[i] = (_Float16)p;
      }
      l_run = l_run * alpha + ps;
      m_run = m_new;
    }
    if (!__all(alpha == 1.f)) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * lg + i, 64);
#pragma unroll
      for (int nb = 0; nb < 32; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nb][i] *= al[i];
    }
    __syncthreads();  // V^T complete
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) {
      const v4i v = *reinterpret_cast<const v4i*>(&vt[(nb * 16 + lq) * VT_STRIDE + lg * 8]);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, __builtin_bit_cast(v8h, v), o[nb], 0, 0, 0);
    }
    __syncthreads();  // V^T free for the next tile
  }

  // per-head sum over the four lanes holding the head
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int h0 = wave * 16;
  if (P.splits == 1) {
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float li = __shfl(l_tot, 4 * lg + i, 64);
      inv[i] = li > 0.f ? 1.f / li : 0.f;
    }
    float* orow = P.out + (size_t)r * ATT_HEADS * LAT_DIM;
#pragma unroll
    for (int nb = 0; nb < 32; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[(size_t)(h0 + 4 * lg + i) * LAT_DIM + nb * 16 + lq] = o[nb][i] * inv[i];
    if (P.lse && lane < 16)
      P.lse[(size_t)r * ATT_HEADS + h0 + lq] = l_tot > 0.f ? m_run * LN2 + logf(l_tot) : -INFINITY;
  } else {
    float* op = P.o_part + ((size_t)r * P.splits + split) * ATT_HEADS * LAT_DIM;
#pragma unroll
    for (int nb = 0; nb < 32; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) op[(size_t)(h0 + 4 * lg + i) * LAT_DIM + nb * 16 + lq] = o[nb][i];
    if (lane < 16) {
      float* mp = P.ml_part + (((size_t)r * P.splits + split) * ATT_HEADS + h0 + lq) * 2;
      mp[0] = m_run;
      mp[1] = l_tot;
    }
  }
}

// Merge the splits of one (row, head): 128 threads x 4 channels.
__global__ __launch_bounds__(128) void k_mla_combine(const MlaPtrs P) {
  const int r = blockIdx.x / ATT_HEADS, h = blockIdx.x % ATT_HEADS;
  const int S = P.splits;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, P.ml_part[(((size_t)r * S + s) * ATT_HEADS + h) * 2]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float* mp = P.ml_part + (((size_t)r * S + s) * ATT_HEADS + h) * 2;
      float f = exp2f(mp[0] - M);
      wsum += f * mp[1];
      float4 v = *reinterpret_cast<const float4*>(P.o_part + (((size_t)r * S + s) * ATT_HEADS + h) * LAT_DIM +
                                                  threadIdx.x * 4);
      acc.x = fmaf(f, v.x, acc.x);
      acc.y = fmaf(f, v.y, acc.y);
      acc.z = fmaf(f, v.z, acc.z);
      acc.w = fmaf(f, v.w, acc.w);
    }
  }
  float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  acc.x *= inv;
  acc.y *= inv;
  acc.z *= inv;
  acc.w *= inv;
  *reinterpret_cast<float4*>(P.out + ((size_t)r * ATT_HEADS + h) * LAT_DIM + threadIdx.x * 4) = acc;
  if (P.lse && threadIdx.x == 0)
    P.lse[(size_t)r * ATT_HEADS + h] = wsum > 0.f ? M * LN2 + logf(wsum) : -INFINITY;
}

MlaPlan plan_mla(int32_t rows, int32_t k) {
  MlaPlan p;
  p.rows = rows;
  int s = (512 + rows - 1) / rows;
  int smax = (k + 15) / 16;  // at least 16 groups (64 tokens) per split
  if (s > smax) s = smax;
  if (s > 32) s = 32;
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
  hipLaunchKernelGGL(k_mla_split, dim3(p.rows * p.splits), dim3(MLA_THREADS), 0, stream, a, P);
  if (hipGetLastError() != hipSuccess) return ISA_ERR_HIP;
  if (p.splits > 1) {
    hipLaunchKernelGGL(k_mla_combine, dim3(p.rows * ATT_HEADS), dim3(128), 0, stream, P);
    if (hipGetLastError() != hipSuccess) return ISA_ERR_HIP;
  }
  return ISA_OK;
}

}  // namespace isa
