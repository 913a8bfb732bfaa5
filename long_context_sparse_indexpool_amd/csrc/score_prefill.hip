// score_prefill.hip -- prefill lightning-indexer scores, a dense int8 MFMA
// contraction with a fused ReLU / head-weight epilogue, gfx950.
//
// Method (pages cited by title): "GLM-5.3 Sparse Attention은 연산량을 줄이지만 HBM
// 수요는 지속된다" (remio.ai), section "GLM-5.3 Sparse Attention이 실제로 바꾸는 것":
// the indexer scores the whole retained history.  "GLM-5.3-Flash vs
// Qwen3.8-Flash-Next" (alltoptrend), section "수렴점 2 — 4배 압축 후 2,048 토큰만
// 유지": 32 heads, keys pooled 4 -> 1 before scoring.  Prefill masking (not on
// the pages; this library's contract): a query at position p sees groups
// g <= floor(p/4), its own group included; later groups get -1.
//
// Scores of Q queries x G groups: [Q*32, 128] x [128, G] int8 -> int32, then
// S[q][g] = sum_h w[q][h] * max(0, acc[q,h][g]).  v_mfma_i32_32x32x32_i8 with a
// query's 32 heads as M and 32 groups as N; four MFMAs cover the 128 channels.
// Each wave keeps 4 queries' operands and head weights (two 16-bit weights per
// register) in registers and streams 32-group key blocks through them, three
// blocks of loads in flight; the accumulators live in VGPRs.  The epilogue is
// two VALU ops per element (max, 24-bit multiply-add with the weight's half
// selected in the instruction) plus one cross-half add, which costs about as
// much issue time as the MFMAs, so each wave issues the MFMAs of its next query
// before the epilogue of the current one.  A workgroup covers 16 queries x
// 4096 groups.  Workgroups are numbered so that every query block of one group
// range lands on the same XCD (dispatch is round-robin over the 8 XCDs): the
// range's 512 KiB of keys is then fetched into that XCD's L2 once and reused
// by all query blocks.
#include "isa_launch.hpp"

namespace isa {

constexpr int PF_THREADS = 256;
constexpr int PF_QW = 4;                      // queries per wave
constexpr int PF_QB = PF_QW * (PF_THREADS / 64);  // queries per workgroup
constexpr int PF_GT = 4096;                   // groups per workgroup
constexpr int N_XCD = 8;

struct PrefillPtrs {
  const int8_t* q;
  const int8_t* hw;
  const int32_t* q_pos;
  const int8_t* pooled;
  const int32_t* bt;
  int32_t* scores;
  int32_t ld;
  int32_t Q;
  int32_t n_qb;
  int32_t n_gr;
  uint32_t* err;
};

__global__ __launch_bounds__(PF_THREADS) void k_prefill_scores(const BatchArgs a, const PrefillPtrs P) {
  __shared__ int32_t pages[PF_GT / PAGE_GRP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: query indices and bases stay scalar
  const int xcd = blockIdx.x % N_XCD;
  const int i = blockIdx.x / N_XCD;
  const int qb = i % P.n_qb;
  const int gr = (i / P.n_qb) * N_XCD + xcd;
  if (gr >= P.n_gr) return;
  const int L = a.lens[0];
  const int G = (L + GROUP - 1) / GROUP;
  const int g0 = gr * PF_GT;
  const int gN = min(G - g0, PF_GT);
  if (tid < PF_GT / PAGE_GRP) {
    pages[tid] = tid * PAGE_GRP < gN ? phys_page(P.bt, a.max_pages, a.num_pages, 0, g0 / PAGE_GRP + tid, P.err)
                                     : -1;
  }

  // this wave's queries: operands, head weights of the accumulator rows, visible range
  v4i qa[PF_QW][4];
  uint32_t wv[PF_QW][8];  // head weights of the accumulator rows, two 16-bit halves per register
  int lastg[PF_QW];
  bool bad = false;
#pragma unroll
  for (int qq = 0; qq < PF_QW; ++qq) {
    int qi = qb * PF_QB + wave * PF_QW + qq;
    bool live = qi < P.Q;
    int qc = live ? qi : 0;
    const v4i* qp = reinterpret_cast<const v4i*>(P.q + (size_t)qc * IDX_HEADS * IDX_DIM + (lane & 31) * IDX_DIM +
                                                 (lane >> 5) * 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) qa[qq][c] = qp[c];
    const int8_t* hp = P.hw + (size_t)qc * IDX_HEADS;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int w = hp[(r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)];
      bad |= (w < 0) | (w > 64);
      wv[qq][r >> 1] = (r & 1) ? (wv[qq][r >> 1] | ((uint32_t)w << 16)) : (uint32_t)w;
    }
    int p = P.q_pos[qc];
    if (live && (p < 0 || p >= L)) {
      bad = true;
      p = -4;
    }
    lastg[qq] = __builtin_amdgcn_readfirstlane(live ? p / GROUP : -2);  // -2: query beyond Q, nothing stored
  }
  if (__any(bad) && lane == 0) report(P.err, ISA_DERR_HEADW_RANGE | ISA_DERR_ROW_RANGE);
  __syncthreads();

  const int8_t* kbase = P.pooled + (lane >> 5) * 64;
  // Loads are unconditional (a group past the range, or on a page outside the
  // pool, reads row 0 and is zeroed by its mask) and the two register buffers
  // alternate by block parity, so each block waits for its own loads only.
  auto load_blk = [&](int blk, v4i (&kb)[4], int& mask) {
    const int gi = blk * 32 + (lane & 31);
    const int gl = min(gi, PF_GT - 1);
    const int pg = pages[gl / PAGE_GRP];
    const bool ok = gi < gN && pg >= 0;
    mask = ok ? -1 : 0;
    const size_t row = ok ? (size_t)pg * PAGE_GRP + gl % PAGE_GRP : 0;
    const v4i* p = reinterpret_cast<const v4i*>(kbase + row * IDX_DIM);
    kb[0] = p[0];
    kb[1] = p[1];
    kb[2] = p[2];
    kb[3] = p[3];
  };
  // each query's score row as a buffer resource (scalar base, 32-bit offsets,
  // stores past the row's end dropped by the range check)
  __amdgpu_buffer_rsrc_t rows[PF_QW];
#pragma unroll
  for (int qq = 0; qq < PF_QW; ++qq) {
    const int qi = min(qb * PF_QB + wave * PF_QW + qq, P.Q - 1);
    rows[qq] = __builtin_amdgcn_make_buffer_rsrc(P.scores + (size_t)qi * P.ld, 0, (g0 + gN) * 4, 0x00020000);
  }
  uint32_t smax = 0;  // largest visible score of this lane (overflow check after the loop)
  // score of the lane's group for query qq from its 32 x 32 accumulator block:
  // the lane holds 16 heads of group l%32; the other 16 are in lane l^32.
  // gb: first group of the block (uniform)
  auto epilogue = [&](const v16i& acc, int qq, int gb) {
    uint32_t s = 0;
#pragma unroll
    for (int r = 0; r < 16; r += 2)  // ReLU <= 2^21: 24-bit multiplies by the packed weights
      s += __umul24((uint32_t)max(acc[r], 0), wv[qq][r >> 1] & 0xFFFFu) +
           __umul24((uint32_t)max(acc[r + 1], 0), wv[qq][r >> 1] >> 16);
    s += __builtin_amdgcn_permlane32_swap(s, s, false, false)[1];  // lanes < 32: + lane l+32
    const int lg = lastg[qq];
    if (lg == -2) return;  // uniform: query beyond Q
    const int g = gb + (lane & 31);
    const bool vis = g <= lg;
    smax = max(smax, vis ? s : 0u);
    if (lane < 32)  // groups past the sequence fall outside the row's range and are dropped
      __builtin_amdgcn_raw_buffer_store_b32(vis ? (int32_t)s : -1, rows[qq], g * 4, 0, 2 /* nontemporal */);
  };
  // one block of 32 groups for the wave's queries; the MFMAs of the next query
  // are issued before the epilogue of the current one, so the matrix core and
  // the VALU work side by side
  auto do_blk = [&](int blk, const v4i (&kb)[4], int mask) {
    const int g = g0 + blk * 32;
    const v4i k[4] = {kb[0] & mask, kb[1] & mask, kb[2] & mask, kb[3] & mask};
    auto mm = [&](int qq) {
      v16i acc = {0};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[qq][c], k[c], acc, 0, 0, 0);
      return acc;
    };
    static_assert(PF_QW % 2 == 0, "queries are pipelined in pairs");
    v16i a0 = mm(0), a1;
#pragma unroll
    for (int qq = 0; qq < PF_QW; qq += 2) {
      a1 = mm(qq + 1);
      epilogue(a0, qq, g);
      if (qq + 2 < PF_QW) a0 = mm(qq + 2);
      epilogue(a1, qq + 1, g);
    }
  };
  const int nblk = (gN + 31) / 32;
  v4i bA[4], bB[4], bC[4];
  int mA, mB, mC;
  load_blk(0, bA, mA);
  __builtin_amdgcn_sched_barrier(0);
  load_blk(1, bB, mB);
  __builtin_amdgcn_sched_barrier(0);
  load_blk(2, bC, mC);
  __builtin_amdgcn_sched_barrier(0);
  for (int blk = 0; blk < nblk; blk += 3) {  // trailing blocks past the range store nothing
    do_blk(blk, bA, mA);
    load_blk(blk + 3, bA, mA);
    do_blk(blk + 1, bB, mB);
    load_blk(blk + 4, bB, mB);
    do_blk(blk + 2, bC, mC);
    load_blk(blk + 5, bC, mC);
  }
  if (__any(lane < 32 && smax > 0x7FFFFFFFu) && lane == 0) report(P.err, ISA_DERR_SCORE_OVERFLOW);  // (lanes >= 32 hold doubled sums)
}

isa_status launch_prefill_scores(const BatchArgs& a, const int8_t* q, const int8_t* hw, const int32_t* q_pos,
                                 int32_t Q, const int8_t* pooled, const int32_t* bt, int32_t* scores,
                                 int32_t ld, uint32_t* err, hipStream_t stream) {
  const int G = (a.lens[0] + GROUP - 1) / GROUP;
  PrefillPtrs P{q, hw, q_pos, pooled, bt, scores, ld, Q, (Q + PF_QB - 1) / PF_QB, (G + PF_GT - 1) / PF_GT, err};
  const int gr_rounds = (P.n_gr + N_XCD - 1) / N_XCD;
  const long long nwg = (long long)gr_rounds * N_XCD * P.n_qb;
  if (nwg > 0x7FFFFFFF) return ISA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k_prefill_scores, dim3((unsigned)nwg), dim3(PF_THREADS), 0, stream, a, P);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

}  // namespace isa
