// latent_fp8.hip -- FP8 latent cache: per-row E4M3 quantisation, gfx950.
//
// Method (pages cited by title): "GLM-5.3-Flash: 하이브리드 희소·선형 어텐션과
// IndexPool·EPD로 1M 컨텍스트를 오픈 소스로 서빙하는 방법" (llm-wiki.hwlabs.dev),
// section "양자화: W8A8와 혼합 캐시": the recent, high-importance cache is kept in
// FP8.  The pages name no FP8 format or scaling (this library's contract): OCP
// E4M3 codes, one fp32 scale per latent row, scale = amax / 448 (1 for a zero
// row), code = round-to-nearest-even of x / scale with the division in fp32.
//
// One wave per token row: each lane loads 16 B (8 channels) of bf16, the wave
// reduces the row's amax, and each lane converts its 8 values with the
// hardware E4M3 conversion (v_cvt_scalef32_pk_fp8_f32, scale 1: nearest-even;
// the quantised values never exceed 448 in magnitude) and stores 8 B.  A
// workgroup of 4 waves covers one page (256 rows) of one sequence, so rows
// past the sequence's end are never touched.
#include "isa_launch.hpp"

namespace isa {

constexpr int FP8_THREADS = 256;

struct Fp8Ptrs {
  const uint16_t* latent;
  const int32_t* bt;
  uint8_t* codes;
  float* scales;
  uint32_t* err;
};

__global__ __launch_bounds__(FP8_THREADS) void k_latent_fp8(const BatchArgs a, const Fp8Ptrs F) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const int tile = blockIdx.x;  // one page of one sequence
  const int b = tile_owner(a, tile);
  const int j = tile - a.tile_start[b];
  const int L = a.lens[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pg = phys_page(F.bt, a.max_pages, a.num_pages, b, j, F.err);
  if (pg < 0) return;
  const int rows = min(PAGE_TOK, L - j * PAGE_TOK);
  bool bad = false;
  for (int r = wave; r < rows; r += FP8_THREADS / 64) {
    const size_t row = (size_t)pg * PAGE_TOK + r;
    const v4i w = reinterpret_cast<const v4i*>(F.latent + row * LAT_DIM)[lane];
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float((uint32_t)w[i] << 16);
      x[2 * i + 1] = __uint_as_float((uint32_t)w[i] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bad |= !isfinite(x[i]);
      amax = fmaxf(amax, fabsf(x[i]));
    }
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float s = amax > 0.f ? amax / 448.f : 1.f;
    uint32_t lo = 0, hi = 0;
    v2s p = {0, 0};
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, x[0] / s, x[1] / s, 1.0f, false);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, x[2] / s, x[3] / s, 1.0f, true);
    lo = __builtin_bit_cast(uint32_t, p);
    p = v2s{0, 0};
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, x[4] / s, x[5] / s, 1.0f, false);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, x[6] / s, x[7] / s, 1.0f, true);
    hi = __builtin_bit_cast(uint32_t, p);
    reinterpret_cast<uint2*>(F.codes + row * LAT_DIM)[lane] = make_uint2(lo, hi);
    if (lane == 0) F.scales[row] = s;
  }
  if (__any(bad) && lane == 0) report(F.err, ISA_DERR_NONFINITE);
}

isa_status launch_latent_fp8(const BatchArgs& a, const uint16_t* latent, const int32_t* bt, uint8_t* codes,
                             float* scales, uint32_t* err, hipStream_t stream) {
  Fp8Ptrs F{latent, bt, codes, scales, err};
  hipLaunchKernelGGL(k_latent_fp8, dim3(a.tile_start[a.batch]), dim3(FP8_THREADS), 0, stream, a, F);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

}  // namespace isa
