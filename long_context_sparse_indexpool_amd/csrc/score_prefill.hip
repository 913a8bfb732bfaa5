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
// A workgroup covers 16 queries x 4096 groups; each of its four waves keeps 4
// queries' operands and head weights in registers.  The 32-group key blocks
// are fetched once per workgroup, by direct-to-LDS loads into a four-slot ring
// (each wave fetches one K step of a block), and every wave reads its operands
// from there: a quarter of the key traffic of per-wave register loads, three
// blocks in flight, no registers spent on prefetch.  The epilogue costs two
// VALU ops per accumulator element (max, 24-bit multiply-add by the head
// weight); the two halves of a query pair's 32 heads meet in one cross-half
// swap, after which each lane finishes one score of one of the two queries.
// The MFMAs of each query are issued before the epilogue of the previous one,
// across block boundaries, so the matrix core and the VALU work side by side.
// Workgroups are numbered so that every query block of one group range lands
// on the same XCD (dispatch is round-robin over the XCDs): the range's
// 512 KiB of keys is then fetched into that XCD's L2 once and reused by all
// query blocks.
#include "isa_launch.hpp"

namespace isa {

constexpr int PF_THREADS = 256;
constexpr int PF_QW = 4;                      // queries per wave
constexpr int PF_QB = PF_QW * (PF_THREADS / 64);  // queries per workgroup
constexpr int PF_GT = 4096;                   // groups per workgroup
constexpr int PF_NS = 4;                      // key blocks staged in LDS (ring slots)
constexpr int PF_KB = 32 * IDX_DIM;           // bytes of one key block (32 groups)

// 16 bytes per lane from global memory straight into LDS: lane l reads
// base + voff (base uniform, in scalar registers) and its bytes land at
// lds + 16 l (lds uniform).  Written out rather than through the builtin:
// the compiler would otherwise guard every later LDS read with a wait for all
// outstanding loads, since it cannot tell ring slots apart.  The instruction
// has no register result; completion is tracked by vmcnt (waited for
// explicitly by the caller).  One wait state separates the M0 write from the
// load that reads it; M0 is declared clobbered, so the compiler keeps nothing
// of its own there across the statement.
__device__ __forceinline__ void load_to_lds16(const int8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N), no wait on the other counters
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// a * b + c on 24-bit unsigned operands in one instruction (the compiler
// otherwise splits it into a multiply and a three-way add)
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// compile-time flag passed to the generic lambdas below
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

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
  int32_t n_xcd;  // XCDs the workgroups are dispatched over, round-robin
  int32_t wide_ok;  // a wave's four score rows fit one buffer resource (16 ld < 2^31)
  uint32_t* err;
};

// Two waves per SIMD (two workgroups per CU) is also what the register budget
// allows; stating it caps a wave at 256 registers, and under that cap the
// compiler keeps the MFMA accumulators in ordinary VGPRs, where the epilogue
// reads them directly (with room for 512 it places them in the accumulation
// registers and copies each element out with an extra VALU move, a quarter of
// the epilogue's instructions).
__global__ __launch_bounds__(PF_THREADS, 2) void k_prefill_scores(const BatchArgs a, const PrefillPtrs P) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: query indices and bases stay scalar
  const int xcd = blockIdx.x % P.n_xcd;
  const int i = blockIdx.x / P.n_xcd;
  const int qb = i % P.n_qb;
  const int gr = (i / P.n_qb) * P.n_xcd + xcd;
  if (gr >= P.n_gr) return;
  const int L = a.lens[0];
  const int G = (L + GROUP - 1) / GROUP;
  const int g0 = gr * PF_GT;
  const int gN = min(G - g0, PF_GT);
  // the range's pages, one per lane (every wave holds the whole table; a
  // block's page is then one uniform read of a lane)
  static_assert(PF_GT / PAGE_GRP == 64 && PAGE_GRP % 32 == 0, "one page per lane; a key block within one page");
  const int pg_lane =
      lane * PAGE_GRP < gN ? phys_page(P.bt, a.max_pages, a.num_pages, 0, g0 / PAGE_GRP + lane, P.err) : -1;

  // this wave's queries: operands, head weights of the accumulator rows, visible range
  v4i qa[PF_QW][4];
  uint32_t wv[PF_QW][16];  // head weights of the accumulator rows
  int lastg[PF_QW];
  bool bad_w = false, bad_p = false;
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
      bad_w |= (w < 0) | (w > 64);
      wv[qq][r] = (uint32_t)w;
    }
    int p = P.q_pos[qc];
    if (live && (p < 0 || p >= L)) {  // nothing of this query is visible
      bad_p = true;
      p = -4;
    }
    lastg[qq] = __builtin_amdgcn_readfirstlane(live ? p / GROUP : -2);  // -2: query beyond Q, nothing stored
  }
  if (__any(bad_w) && lane == 0) report(P.err, ISA_DERR_HEADW_RANGE);
  if (__any(bad_p) && lane == 0) report(P.err, ISA_DERR_ROW_RANGE);
  __syncthreads();

  // Key blocks (32 groups x 128 B) are staged once per workgroup in a ring of
  // PF_NS LDS slots by direct-to-LDS loads: wave w fetches K step w of a block
  // (lane l: group l%32, channels 64(l/32) + 16w .. +15), which lands at slot
  // + 1024w + 16l, so every wave's operand read of K step c is one contiguous
  // KiB.  A block lies within one page, so its address is a uniform base plus
  // a fixed per-lane offset.  Loads are unconditional: groups past the range
  // read the rest of their page (a block past the last page, or a page outside
  // the pool, reads page 0) -- all inside the pool; their scores are masked
  // out of the overflow check and fall outside the row's buffer range, and a
  // page outside the pool has already been reported as an error.
  __shared__ __attribute__((aligned(16))) int8_t ring[PF_NS][PF_KB];
  const uint32_t key_off = (lane & 31) * IDX_DIM + (lane >> 5) * 64 + wave * 16;
  auto issue = [&](int blk) {
    const int pg = __builtin_amdgcn_readlane(pg_lane, min(blk, PF_GT / 32 - 1) >> 1);
    const size_t row0 = pg >= 0 ? (size_t)pg * PAGE_GRP + (blk & 1) * 32 : 0;
    load_to_lds16(P.pooled + row0 * IDX_DIM, key_off,
                  (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int8_t*)&ring[blk % PF_NS][wave * 1024]);
  };
  auto read_blk = [&](int blk, v4i (&k)[4]) {
    const int8_t* src = &ring[blk % PF_NS][lane * 16];
#pragma unroll
    for (int c = 0; c < 4; ++c) k[c] = *reinterpret_cast<const v4i*>(src + c * 1024);
  };
  // each query's score row as a buffer resource (scalar base, 32-bit offsets,
  // stores past the row's end dropped by the range check; a query beyond Q
  // gets an empty range, so nothing of it is stored)
  __amdgpu_buffer_rsrc_t rows[PF_QW];
#pragma unroll
  for (int qq = 0; qq < PF_QW; ++qq) {
    const int qi = qb * PF_QB + wave * PF_QW + qq;
    rows[qq] = __builtin_amdgcn_make_buffer_rsrc(P.scores + (size_t)min(qi, P.Q - 1) * P.ld, 0,
                                                 qi < P.Q ? (g0 + gN) * 4 : 0, 0x00020000);
  }
  // visibility bound per query pair: lanes < 32 carry the pair's first query,
  // lanes >= 32 its second (the layout of a pair's finished scores)
  int lgp[PF_QW / 2];
#pragma unroll
  for (int pr = 0; pr < PF_QW / 2; ++pr) {
    // (both bounds taken as uniform values first: a per-lane choice between
    // two array elements would otherwise be folded into a dynamic index, which
    // moves the array out of registers)
    const int l0 = __builtin_amdgcn_readfirstlane(lastg[2 * pr]), l1 = __builtin_amdgcn_readfirstlane(lastg[2 * pr + 1]);
    lgp[pr] = min(lane < 32 ? l0 : l1, g0 + gN - 1);  // range clamp: see the loop
  }
  const uint32_t oob_lo = lane < 32 ? 0u : 0x80000000u;  // beyond every row's range
  const uint32_t oob_hi = lane < 32 ? 0x80000000u : 0u;
  // Fast blocks store through one resource over this wave's four score rows:
  // after the cross-half swap lane l holds query 2pr + l / 32's score of group
  // l % 32, so each lane stores exactly one word (no half pushed out of range).
  // Rows past Q lie beyond the resource's range and are dropped.
  const int qw0 = qb * PF_QB + wave * PF_QW;
  const int nrow_w = min(max(P.Q - qw0, 0), PF_QW);
  // (base and size passed through readfirstlane: the compiler otherwise keeps
  // this resource in vector registers and wraps every store in a loop over
  // its distinct values)
  const uint64_t wbase = (uint64_t)(uintptr_t)(P.scores + (size_t)(nrow_w > 0 ? qw0 : 0) * P.ld);
  const __amdgpu_buffer_rsrc_t wrows = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(wbase >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)wbase)),
      0, __builtin_amdgcn_readfirstlane(P.wide_ok ? nrow_w * P.ld * 4 : 0), 0x00020000);
  uint32_t voff_w[PF_QW / 2];
#pragma unroll
  for (int pr = 0; pr < PF_QW / 2; ++pr) voff_w[pr] = ((2 * pr + (lane >> 5)) * (uint32_t)P.ld + (lane & 31)) * 4u;
  // leading blocks whose 32 groups are all inside the range and visible to all
  // four of this wave's queries: they need no mask (uniform)
  const int minlast = min(min(lastg[0], lastg[1]), min(lastg[2], lastg[3]));
  const int nfast = P.wide_ok ? max(0, min(gN / 32, (minlast - g0 + 1) / 32)) : 0;
  uint32_t smax = 0;  // largest visible score of this lane (overflow check after the loop)
  // this lane's share of query qq's score of group l%32 from its 32 x 32
  // accumulator block: the lane holds 16 of the 32 heads, lane l^32 the others
  auto partial = [&](const v16i& acc, int qq) {
    uint32_t s = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s = mad_u24((uint32_t)max(acc[r], 0), wv[qq][r], s);  // ReLU <= 2^21
    return s;
  };
  // scores of the query pair (2pr, 2pr + 1) for the block's 32 groups (gb
  // uniform): one cross-half swap leaves the first query's sums in lanes < 32
  // and the second's in lanes >= 32, so every lane finishes one score.  A
  // block without masking (fast) stores it once through the wave's four-row
  // resource, its first group's offset added as the uniform scalar offset.
  // Otherwise both per-row stores go out from every lane, each half's offset
  // pushed out of the other row's range (uniform resources, no per-lane
  // branch), groups past the query's position are stored as -1, and groups
  // past the sequence fall outside the row's range and are dropped.
  auto finish = [&](uint32_t s0, uint32_t s1, int pr, int gb, auto fast) {
    const auto sw = __builtin_amdgcn_permlane32_swap(s0, s1, false, false);
    const uint32_t s = sw[0] + sw[1];
    if constexpr (decltype(fast)::value) {
      smax = max(smax, s);
      __builtin_amdgcn_raw_buffer_store_b32((int32_t)s, wrows, voff_w[pr], gb * 4, 2 /* nontemporal */);
    } else {
      const int g = gb + (lane & 31);
      const bool vis = g <= lgp[pr];
      smax = max(smax, vis ? s : 0u);
      const int32_t v = vis ? (int32_t)s : -1;
      __builtin_amdgcn_raw_buffer_store_b32(v, rows[2 * pr], (g * 4) | oob_lo, 0, 2 /* nontemporal */);
      __builtin_amdgcn_raw_buffer_store_b32(v, rows[2 * pr + 1], (g * 4) | oob_hi, 0, 2 /* nontemporal */);
    }
  };
  auto mm = [&](const v4i (&k)[4], int qq) {
    v16i acc = {0};
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[qq][c], k[c], acc, 0, 0, 0);
    return acc;
  };
  // Software pipeline over (block, query): the MFMAs of each query are issued
  // before the epilogue of the previous one, so the matrix core and the VALU
  // work side by side; the last query of a block is finished in the next
  // block.  At most two accumulators are live at any point.
  static_assert(PF_QW == 4, "the pipeline below is written for four queries per wave");
  v16i pend;       // accumulator of the previous block's last query
  uint32_t s2 = 0;  // partial of the previous block's third query
  // fprev / fcur: whether the previous / this block is a fast one
  auto do_blk = [&](int blk, const v4i (&k)[4], bool first, auto fprev, auto fcur) {
    const int g = g0 + blk * 32;
    v16i x = mm(k, 0);
    if (!first) finish(s2, partial(pend, 3), 1, g - 32, fprev);
    v16i y = mm(k, 1);
    const uint32_t s0 = partial(x, 0);
    x = mm(k, 2);
    finish(s0, partial(y, 1), 0, g, fcur);
    pend = mm(k, 3);
    s2 = partial(x, 2);
  };
  const Flag<true> FAST;
  const Flag<false> MASKED;
  // Block b: wait for this wave's load of block b, meet the other waves (their
  // quarters of the block are then in LDS, and every wave is done with the
  // slot of block b - 1), refill that slot with block b + PF_NS - 1, compute.
  // The compiler does not track direct-to-LDS loads, so the waits are explicit:
  // vmcnt counts loads and stores in issue order, and the load of block b is
  // followed by PF_NS - 2 later loads and the score stores of the blocks in
  // between.  The counts take the fewest stores a block can issue (one per
  // finished pair in a fast block: one in block 0, two in every later block;
  // a masked block issues twice as many); a count below the true one only
  // waits longer.
  static_assert(PF_NS == 4, "the wait counts below are written for four slots");
  const int nblk = (gN + 31) / 32;
  v4i kb[4];
#pragma unroll
  for (int b = 0; b < PF_NS - 1; ++b) issue(b);
  wait_vmcnt<PF_NS - 2>();
  lds_barrier();
  asm volatile("" ::: "memory");
  issue(PF_NS - 1);
  read_blk(0, kb);
  if (nfast > 0)
    do_blk(0, kb, true, MASKED, FAST);
  else
    do_blk(0, kb, true, MASKED, MASKED);
  auto next = [&](int blk) {
    // later loads (PF_NS - 2) + fewest stores of the blocks issued after block
    // blk's load: blocks 0 .. blk-1 for blk < PF_NS (block 0 one store, the
    // others two), the PF_NS - 1 blocks before it otherwise
    if (blk >= PF_NS)
      wait_vmcnt<(PF_NS - 2) + 2 * (PF_NS - 1)>();
    else if (blk == 1)
      wait_vmcnt<(PF_NS - 2) + 1>();
    else if (blk == 2)
      wait_vmcnt<(PF_NS - 2) + 1 + 2>();
    else
      wait_vmcnt<(PF_NS - 2) + 1 + 2 + 2>();
    lds_barrier();
    asm volatile("" ::: "memory");
    issue(blk + PF_NS - 1);
    read_blk(blk, kb);
  };
  // the fast blocks lead; one loop per kind, so no path merges inside a loop
  // (a merge would copy the pending accumulator every block)
  int blk = 1;
  for (; blk < nfast; ++blk) {
    next(blk);
    do_blk(blk, kb, false, FAST, FAST);
  }
  if (blk == nfast && blk < nblk) {
    next(blk);
    do_blk(blk, kb, false, FAST, MASKED);
    ++blk;
  }
  for (; blk < nblk; ++blk) {
    next(blk);
    do_blk(blk, kb, false, MASKED, MASKED);
  }
  if (blk - 1 < nfast)
    finish(s2, partial(pend, 3), 1, g0 + (blk - 1) * 32, FAST);
  else
    finish(s2, partial(pend, 3), 1, g0 + (blk - 1) * 32, MASKED);
  if (__any(smax > 0x7FFFFFFFu) && lane == 0) report(P.err, ISA_DERR_SCORE_OVERFLOW);
  // columns past the sequence's last group, up to the row stride, are not
  // candidates: the last group range writes them as -1 for its queries
  if (gr == P.n_gr - 1) {
    for (int qq = 0; qq < PF_QW; ++qq) {
      const int qi = qb * PF_QB + wave * PF_QW + qq;
      if (qi >= P.Q) break;  // uniform
      int32_t* row = P.scores + (size_t)qi * P.ld;
      for (int c = G + lane; c < P.ld; c += 64) row[c] = -1;
    }
  }
}

isa_status launch_prefill_scores(const BatchArgs& a, const int8_t* q, const int8_t* hw, const int32_t* q_pos,
                                 int32_t Q, const int8_t* pooled, const int32_t* bt, int32_t* scores,
                                 int32_t ld, uint32_t* err, hipStream_t stream) {
  const int G = (a.lens[0] + GROUP - 1) / GROUP;
  const int nx = device_info().n_xcd;
  const int wide_ok = (long long)ld * 4 * PF_QW < (1LL << 31) ? 1 : 0;
  PrefillPtrs P{q,  hw, q_pos, pooled, bt, scores, ld, Q, (Q + PF_QB - 1) / PF_QB, (G + PF_GT - 1) / PF_GT, nx, wide_ok,
                err};
  const int gr_rounds = (P.n_gr + nx - 1) / nx;
  const long long nwg = (long long)gr_rounds * nx * P.n_qb;
  if (nwg > 0x7FFFFFFF) return ISA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k_prefill_scores, dim3((unsigned)nwg), dim3(PF_THREADS), 0, stream, a, P);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

}  // namespace isa
