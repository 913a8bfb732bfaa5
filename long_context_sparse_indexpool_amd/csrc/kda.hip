// kda.hip -- one decode step of a linear-attention (KDA) layer, gfx950.
//
// Method (pages cited by title): "GLM-5.3-Flash: 하이브리드 희소·선형 어텐션과
// IndexPool·EPD로 1M 컨텍스트를 오픈 소스로 서빙하는 방법" (llm-wiki.hwlabs.dev),
// section "선형 어텐션: O(1) KV 메모리": a fixed-size state matrix takes the delta
// update S_t = S_{t-1} - beta k (k^T S_{t-1}) + beta k v^T; section "양자화: W8A8와
// 혼합 캐시": the shared state matrix stays BF16.  "GLM-5.3-Flash vs
// Qwen3.8-Flash-Next" (alltoptrend), section "왜 linear 레이어가 절반 이상을
// 차지할까": KDA applies its decay gate channel by channel.  Reading (this
// library's contract): per head, with the state S [128][128] (row = key
// channel, column = value channel),
//   S' = diag(alpha) S;  u = S'^T k;  S'' = S' + beta k (v - u)^T;  o = S''^T q;
// S is stored back in bf16, rounded to nearest even.
//
// HBM-bound: 32 KiB of state in and out per head and token.  One 256-thread
// workgroup per (sequence, head): thread t owns value columns 2(t%64), +1 and
// key rows 32(t/64) .. +31, so each load instruction of a wave reads one whole
// 256-B state row; the two column reductions (u, then o) combine the four row
// quarters through LDS.  Arithmetic in fp32.
#include "isa_launch.hpp"

namespace isa {

constexpr int KDA_D = 128;
constexpr int KDA_THREADS = 256;

struct KdaPtrs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* alpha;
  const float* beta;
  uint16_t* state;
  float* out;
  uint32_t* err;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite inputs (checked by the caller)
}

__global__ __launch_bounds__(KDA_THREADS) void k_kda_step(const KdaPtrs P) {
  __shared__ float ks[KDA_D], qs[KDA_D], as[KDA_D];
  __shared__ float red[4][KDA_D];
  const int unit = blockIdx.x, t = threadIdx.x;
  const int cp = t & 63, qd = t >> 6;  // columns 2cp, 2cp+1; rows 32qd .. +31
  if (t < KDA_D) {
    ks[t] = bf16_to_f32(P.k[(size_t)unit * KDA_D + t]);
    qs[t] = bf16_to_f32(P.q[(size_t)unit * KDA_D + t]);
    as[t] = P.alpha[(size_t)unit * KDA_D + t];
  }
  const uint32_t vw = reinterpret_cast<const uint32_t*>(P.v + (size_t)unit * KDA_D)[cp];
  const float v0 = bf16_to_f32(vw & 0xFFFFu), v1 = bf16_to_f32(vw >> 16);
  const float beta = P.beta[unit];
  uint32_t* st = reinterpret_cast<uint32_t*>(P.state + (size_t)unit * KDA_D * KDA_D);
  float s0[32], s1[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t w = st[(32 * qd + i) * (KDA_D / 2) + cp];
    s0[i] = bf16_to_f32(w & 0xFFFFu);
    s1[i] = bf16_to_f32(w >> 16);
  }
  __syncthreads();
  // decay, then what the key retrieves from the decayed state
  float u0 = 0.f, u1 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * qd + i;
    s0[i] *= as[row];
    s1[i] *= as[row];
    u0 = fmaf(ks[row], s0[i], u0);
    u1 = fmaf(ks[row], s1[i], u1);
  }
  red[qd][2 * cp] = u0;
  red[qd][2 * cp + 1] = u1;
  __syncthreads();
  u0 = ((red[0][2 * cp] + red[1][2 * cp]) + red[2][2 * cp]) + red[3][2 * cp];
  u1 = ((red[0][2 * cp + 1] + red[1][2 * cp + 1]) + red[2][2 * cp + 1]) + red[3][2 * cp + 1];
  const float d0 = beta * (v0 - u0), d1 = beta * (v1 - u1);
  // delta update and the read-out
  float o0 = 0.f, o1 = 0.f;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * qd + i;
    s0[i] = fmaf(ks[row], d0, s0[i]);
    s1[i] = fmaf(ks[row], d1, s1[i]);
    bad |= !isfinite(s0[i]) | !isfinite(s1[i]);
    o0 = fmaf(qs[row], s0[i], o0);
    o1 = fmaf(qs[row], s1[i], o1);
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) st[(32 * qd + i) * (KDA_D / 2) + cp] = f32_to_bf16_rne(s0[i]) | (f32_to_bf16_rne(s1[i]) << 16);
  __syncthreads();  // every thread has read red[] for u
  red[qd][2 * cp] = o0;
  red[qd][2 * cp + 1] = o1;
  __syncthreads();
  if (qd == 0) {
    float* op = P.out + (size_t)unit * KDA_D;
    op[2 * cp] = ((red[0][2 * cp] + red[1][2 * cp]) + red[2][2 * cp]) + red[3][2 * cp];
    op[2 * cp + 1] = ((red[0][2 * cp + 1] + red[1][2 * cp + 1]) + red[2][2 * cp + 1]) + red[3][2 * cp + 1];
  }
  if (__any(bad) && (t & 63) == 0) report(P.err, ISA_DERR_NONFINITE);
}

isa_status launch_kda_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                           const float* beta, uint16_t* state, float* out, int32_t n, uint32_t* err,
                           hipStream_t stream) {
  KdaPtrs P{q, k, v, alpha, beta, state, out, err};
  hipLaunchKernelGGL(k_kda_step, dim3(n), dim3(KDA_THREADS), 0, stream, P);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

}  // namespace isa
