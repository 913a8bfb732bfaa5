// indexer_decode.hip -- decode-time lightning-indexer scoring and exact top-k
// group selection, for gfx950.
//
// Method (pages cited by title): "GLM-5.3 Sparse Attention은 연산량을 줄이지만 HBM
// 수요는 지속된다" (remio.ai), section "GLM-5.3 Sparse Attention이 실제로 바꾸는 것":
// the indexer scores every earlier position and keeps the top-k; below the
// budget attention stays dense.  "GLM-5.3-Flash vs Qwen3.8-Flash-Next" (alltoptrend),
// section "수렴점 2 — 4배 압축 후 2,048 토큰만 유지": a 32-head indexer over keys pooled
// 4 -> 1, top 512 blocks of 4 tokens.  Score of a pooled group (the pages print
// no formula; this library's contract): S = sum_h w_h * max(0, q_h . k).
//
// Two launches, no cross-workgroup synchronisation inside either (on this
// 8-XCD part a device-scope fence writes back the whole L2, which cost more
// than the streaming itself; the kernel boundary gives coherence for free).
//
// k_indexer_score: one workgroup per work tile of 8192 pooled groups (128
// pages) of one sequence, one workgroup per CU; a batch that would make fewer
// tiles than CUs uses tiles of 4096 or 2048 groups.  Its sixteen waves stream the
// tile's int8 keys straight from HBM into v_mfma_i32_32x32x32_i8 operands --
// the 32 indexer heads are M (the query stays in registers), 32 groups are N,
// four MFMAs span the 128 channels, each lane loading 64 contiguous bytes of
// one key.  Waves take 32-group chunks from an LDS counter (two chunks of
// loads in flight per wave), so a wave that the memory system serves slowly
// does not hold back the workgroup's epilogue.  The epilogue applies ReLU and the head weights exactly
// in u32 (every partial stays below 2^32) and adds the two lane halves.  The
// workgroup then keeps only candidates that can still reach the global top-k:
// it histograms its scores by an 11-bit monotone key, finds the bin of its own
// k-th best, and writes every candidate from that bin up into a per-tile list
// ordered by descending bin, plus the (bin, count) pairs of those bins.
//
// k_indexer_select: one workgroup per sequence.  It sums the tiles' (bin,
// count) pairs into an LDS histogram, finds the global boundary bin, takes
// every candidate above it, resolves the boundary bin exactly on (score, -id)
// keys, sorts the k ids ascending and writes them.  No state outlives a call:
// the workspace holds only what the scoring kernel wrote in the same call.
#include "isa_launch.hpp"
#include "select_device.hpp"

namespace isa {

constexpr int DEC_THREADS = 1024;
constexpr int SEL_THREADS = 512;
constexpr int SEL_CAND = 2048;           // boundary candidates resolved in LDS
constexpr int SEL_LDS_PAIRS = 8192;      // (bin, count) pairs fetched into LDS in the first round
constexpr int SEL_LDS_HEAD = 4096;       // candidate-list entries fetched into LDS in the first round
constexpr int SEL_BUCKETS = 1024;        // id buckets of the final ascending order
constexpr int SEL_REFINE = 128;          // boundary lists longer than this take one more histogram level

struct DecodePtrs {
  const int8_t* q;
  const int8_t* hw;
  const int8_t* pooled;
  const int32_t* bt;
  uint2* tile_meta;     // [ntiles] (candidates, pairs)
  uint32_t* tile_pairs; // [ntiles][PAIR_CAP] (bin << 16 | count), descending bins
  uint64_t* tile_list;  // [ntiles][TILE_CAP] (score << 32 | group), descending bins
  int32_t* out_idx;     // [B][k]
  int32_t* out_count;   // [B]
  int32_t* scores_out;  // [B][ld] or null
  int32_t ld_scores;
  uint32_t* err;
};

__global__ __launch_bounds__(DEC_THREADS) void k_indexer_score(const BatchArgs a, const DecodePtrs P) {
  __shared__ uint32_t sc[TILE_CAP];   // tile scores
  __shared__ uint32_t hist[NBINS];  // tile histogram -> emission cursors
  __shared__ uint32_t scr[SCR_WORDS];
  __shared__ int32_t pages[TILE_CAP / PAGE_GRP];
  __shared__ uint32_t chunk_ctr;
  // per wave, one 32-group chunk on its way from the load layout to the MFMA
  // layout: piece j (16 B) of row r at 16 (8r + (j ^ ((r >> 1) & 7)))
  __shared__ __attribute__((aligned(16))) v4i stage[DEC_THREADS / 64][32 * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int b = tile_owner(a, tile);
  const int L = a.lens[b];
  const int G = (L + GROUP - 1) / GROUP;
  const uint32_t K = (uint32_t)a.k;
  const int tg = a.tile_g;  // groups per tile of this call (a multiple of 64, 2048 .. 8192)
  // The tiles of a pair (local indices 2i, 2i + 1) that lies wholly inside
  // the sequence move tile_skew groups from the one on an odd-numbered XCD to
  // the one on an even-numbered XCD (the grid is one workgroup per tile,
  // dispatched round-robin over the XCDs, so global tile parity is XCD parity).
  const int jt = tile - a.tile_start[b];  // tile within the sequence
  const bool pair_full = ((jt | 1) + 1) * tg <= G;
  const int sg = pair_full ? (((tile - (jt & 1)) & 1) == 0 ? a.tile_skew : -a.tile_skew) : 0;  // first tile's extra
  const int g0 = jt * tg + ((jt & 1) ? sg : 0);
  const int tsz = (jt & 1) ? tg - sg : tg + sg;  // groups of this tile (fewer where the sequence ends)
  const int gN = min(G - g0, tsz);
  const bool dense = G <= (int)K;

  if (dense && P.scores_out == nullptr) {  // at most k groups: select them all
    for (int i = tid; i < (int)K; i += DEC_THREADS) P.out_idx[(size_t)b * K + i] = i < G ? i : -1;
    if (tid == 0) P.out_count[b] = G;
    return;
  }

  for (int i = tid; i < NBINS; i += DEC_THREADS) hist[i] = 0;
  if (tid == 0) chunk_ctr = 2 * (DEC_THREADS / 64);
  if (tid < tsz / PAGE_GRP) {
    const int jp = (g0 / PAGE_GRP) + tid;
    pages[tid] = (tid * PAGE_GRP < gN) ? phys_page(P.bt, a.max_pages, a.num_pages, b, jp, P.err) : -1;
  }

  // Query as the MFMA A operand: lane -> head lane%32, channels (lane/32)*64 + 16c .. +15.
  v4i qa[4];
  {
    const v4i* qp = reinterpret_cast<const v4i*>(P.q + (size_t)b * IDX_HEADS * IDX_DIM + (lane & 31) * IDX_DIM +
                                                 (lane >> 5) * 64);
    qa[0] = qp[0];
    qa[1] = qp[1];
    qa[2] = qp[2];
    qa[3] = qp[3];
  }
  // Head weight of each accumulator row this lane holds: row(i) = 8(i/4) + 4(lane/32) + i%4.
  uint32_t wv[16];
  {
    const int8_t* hp = P.hw + (size_t)b * IDX_HEADS;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int w = hp[(i >> 2) * 8 + (lane >> 5) * 4 + (i & 3)];
      bad |= (w < 0) | (w > 64);
      wv[i] = (uint32_t)w;
    }
    if (__any(bad) && tid == 0) report(P.err, ISA_DERR_HEADW_RANGE);
  }
  __syncthreads();

  // ---- stream the tile: waves take 32-group chunks from an LDS counter ----
  const int nch = tsz / 32;  // chunks of the tile (at least 2 per wave)
  constexpr int NW = DEC_THREADS / 64;
  // A chunk (32 groups, 4 KiB, inside one page) is read as four 1-KiB
  // stretches, lane l taking 16 B at 16 l of each, with non-temporal loads:
  // load q brings piece l % 8 of row 8q + l / 8.  Contiguous wave-wide loads
  // stream faster than the MFMA layout read straight from memory (32 rows per
  // load).  Loads are unconditional (a chunk past the end, or on a page
  // outside the pool, reads the pool's first chunk and is zeroed by its mask),
  // so the compiler waits for exactly the chunk it consumes.
  auto load_chunk = [&](int c, v4i (&kb)[4], int& mask) {
    const int cl = min(c, nch - 1) * 32;
    const int pg = pages[cl / PAGE_GRP];
    const int gl = cl + (lane & 31);  // the group this lane holds in the MFMA layout
    mask = c < nch && gl < gN && pg >= 0 ? -1 : 0;
    const size_t row0 = c < nch && pg >= 0 ? (size_t)pg * PAGE_GRP + (cl % PAGE_GRP) : 0;
    const v4i* p = reinterpret_cast<const v4i*>(P.pooled + row0 * IDX_DIM) + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) kb[q] = __builtin_nontemporal_load(p + q * 64);
  };
  bool overflow = false;
  auto compute = [&](int c, v4i (&kb)[4], int mask) {
    // through the wave's LDS slot into the MFMA layout: lane l takes row l % 32,
    // pieces 4(l / 32) + q (channels 64(l / 32) + 16q .. +15); the slot's
    // swizzle keeps both the stores and the loads free of bank conflicts, and
    // the wave's LDS accesses complete in order, so the slot needs no barrier
    v4i* st = stage[wave];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * q + (lane >> 3), j = lane & 7;
      st[8 * r + (j ^ ((r >> 1) & 7))] = kb[q];
    }
    v4i kr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = lane & 31, j = 4 * (lane >> 5) + q;
      kr[q] = st[8 * r + (j ^ ((r >> 1) & 7))];
    }
    v16i acc = {0};
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[q], kr[q] & mask, acc, 0, 0, 0);
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += __umul24((uint32_t)max(acc[i], 0), wv[i]);  // ReLU <= 128 * 127 * 128 < 2^24: 24-bit multiply
    s += __builtin_amdgcn_permlane32_swap(s, s, false, false)[1];  // lanes < 32: + lane l+32
    const int gl = c * 32 + (lane & 31);
    if (lane < 32) {
      bool valid = gl < gN;
      sc[gl] = valid ? s : INVALID_SCORE;
      if (valid && !dense) atomicAdd(&hist[score_bin(s)], 1u);  // histogram built while streaming
      overflow |= valid && s > 0x7FFFFFFFu;
      if (P.scores_out && valid) P.scores_out[(size_t)b * P.ld_scores + g0 + gl] = (int32_t)s;
    }
  };
  auto grab = [&]() -> int {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(&chunk_ctr, 1u);
    return __builtin_amdgcn_readfirstlane((int)v);
  };
  // two register buffers; a chunk is grabbed when the buffer holding the
  // previous one is consumed, and the counter only grows, so a wave's current
  // chunk in A always precedes the one in B
  v4i bA[4], bB[4];
  int mA, mB;
  int cA = wave, cB = wave + NW;
  load_chunk(cA, bA, mA);
  __builtin_amdgcn_sched_barrier(0);
  load_chunk(cB, bB, mB);
  __builtin_amdgcn_sched_barrier(0);
  for (;;) {
    if (cA >= nch) break;
    {
      const int nA = grab();
      compute(cA, bA, mA);
      cA = nA;
      load_chunk(cA, bA, mA);
    }
    if (cB >= nch) break;
    {
      const int nB = grab();
      compute(cB, bB, mB);
      cB = nB;
      load_chunk(cB, bB, mB);
    }
  }
  if (__any(overflow) && lane == 0) report(P.err, ISA_DERR_SCORE_OVERFLOW);
  // The epilogue's barriers order LDS only: waiting for global memory here
  // (the last chunks' discarded loads, the pair and meta stores) would add its
  // latency to every tile.
  lds_barrier();

  if (dense) {  // only reached when scores were requested
    for (int i = tid; i < (int)K; i += DEC_THREADS) P.out_idx[(size_t)b * K + i] = i < G ? i : -1;
    if (tid == 0) P.out_count[b] = G;
    return;
  }

  // ---- local candidates: every score in a bin >= the bin of this tile's k-th best ----
  // Thread t owns bins NBINS-2t-1 (higher) and NBINS-2t-2, so ascending threads
  // walk the bins in descending order.  One packed prefix sum over the threads
  // gives, for every bin, the candidates and the nonzero bins above it; the
  // kept bins (>= the boundary) are a prefix of that order, so these are also
  // their emission offsets and (bin, count) pair positions.
  constexpr int PER = (TILE_CAP + DEC_THREADS - 1) / DEC_THREADS;  // scores per thread of the largest tile
  static_assert(NBINS == 2 * DEC_THREADS, "two bins per thread");
  static_assert(TILE_CAP < 65536 && NBINS < 65536, "counts and nonzero bins share one word");
  const int hb = NBINS - 2 * tid;
  const uint32_t c_hi = hist[hb - 1], c_lo = hist[hb - 2];
  const uint32_t local = c_hi + c_lo, nzl = (c_hi != 0u) + (c_lo != 0u);
  const uint32_t packed = local | (nzl << 16);
  const uint32_t xin = wave_inclusive_scan(packed);
  if (lane == 63) scr[wave] = xin;
  lds_barrier();
  uint32_t above = xin - packed, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t_ = scr[w];
    all += t_;
    if (w < wave) above += t_;
  }
  const uint32_t run_hi = above & 0xFFFFu, pz_hi = above >> 16;
  const uint32_t total = all & 0xFFFFu;
  if (tid == 0 && total < K) {  // at most k valid scores: keep them all
    scr[SCR_RES] = 0;
    scr[SCR_RES + 1] = total;
    scr[SCR_RES + 2] = all >> 16;
  }
  if (total >= K && run_hi < K && run_hi + local >= K) {  // the boundary bin is one of this thread's
    const bool in_hi = run_hi + c_hi >= K;
    scr[SCR_RES] = (uint32_t)(in_hi ? hb - 1 : hb - 2);
    scr[SCR_RES + 1] = in_hi ? run_hi + c_hi : run_hi + local;
    scr[SCR_RES + 2] = in_hi ? pz_hi + 1u : pz_hi + nzl;
  }
  lds_barrier();
  const int blo = (int)scr[SCR_RES];
  uint32_t* pairs = P.tile_pairs + (size_t)tile * PAIR_CAP;
  // kept bins, descending: (bin, count) pairs and emission cursors
  if (hb - 1 >= blo) {
    if (c_hi) pairs[pz_hi] = ((uint32_t)(hb - 1) << 16) | c_hi;
    hist[hb - 1] = run_hi;
  }
  if (hb - 2 >= blo) {
    if (c_lo) pairs[pz_hi + (c_hi != 0u)] = ((uint32_t)(hb - 2) << 16) | c_lo;
    hist[hb - 2] = run_hi + c_hi;
  }
  if (tid == 0) P.tile_meta[tile] = make_uint2(scr[SCR_RES + 1], scr[SCR_RES + 2]);
  lds_barrier();
  uint64_t* list = P.tile_list + (size_t)tile * TILE_CAP;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int e = tid + j * DEC_THREADS;
    if (e >= tsz) break;  // uniform
    uint32_t s = sc[e];
    if (s == INVALID_SCORE) continue;
    int bin = score_bin(s);
    if (bin < blo) continue;
    uint32_t slot = atomicAdd(&hist[bin], 1u);
    list[slot] = ((uint64_t)s << 32) | (uint32_t)(g0 + e);
  }
}

// Index j with off[j] <= i < off[j+1] (off ascending, n entries + sentinel).
__device__ __forceinline__ int owner_of(const uint32_t* off, int n, uint32_t i) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Per sequence: merge the tiles' candidates into the exact top k.
//  1. one batch of loads, all issued before any is used: every tile's (kept,
//     pairs), the head of its (bin, count) list and the head of its candidate
//     list (both lists share the descending bin order); the pairs are summed
//     into an LDS histogram.  Longer pair lists (a tile spread over many bins)
//     take one more, flat, round;
//  2. the global boundary bin and, per tile, how many candidates lie above it
//     and in it;
//  3. the candidates come from the LDS list heads (global memory only for a
//     tile with more candidates than its head holds);
//  4. the boundary candidates are ranked by (score, -id) -- all-pairs counting
//     in LDS, or radix select when there are too many -- and the k ids are
//     placed in ascending order by counting, straight into the output row.
__global__ __launch_bounds__(SEL_THREADS) void k_indexer_select(const BatchArgs a, const DecodePtrs P) {
  __shared__ __attribute__((aligned(16))) uint32_t lpairs[SEL_LDS_PAIRS];  // later: the sub-boundary keys
  __shared__ uint64_t lhead[SEL_LDS_HEAD];
  __shared__ uint32_t npr[TILE_MAX_PER_SEQ];
  __shared__ uint32_t ovf_off[TILE_MAX_PER_SEQ + 1];
  __shared__ uint32_t sure_off[TILE_MAX_PER_SEQ + 1];
  __shared__ uint32_t bnd_off[TILE_MAX_PER_SEQ + 1];
  __shared__ uint32_t ngt[TILE_MAX_PER_SEQ];
  __shared__ uint32_t nbd[TILE_MAX_PER_SEQ];
  __shared__ __attribute__((aligned(16))) uint64_t cand[SEL_CAND + 2];
  __shared__ uint32_t sel[MAX_K];
  __shared__ __attribute__((aligned(16))) uint32_t h256[256];
  __shared__ uint32_t scr[SCR_WORDS];
  __shared__ uint32_t bcnt[SEL_BUCKETS];
  __shared__ uint32_t bbase[SEL_BUCKETS];
  __shared__ uint32_t bstage[MAX_K];
  __shared__ __attribute__((aligned(16))) uint32_t shist[NBINS];  // candidates per score bin over the tiles

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NWV = SEL_THREADS / 64;
  const int b = blockIdx.x;
  const int G = (a.lens[b] + GROUP - 1) / GROUP;
  const uint32_t K = (uint32_t)a.k;
  if (G <= (int)K) return;  // dense row: written by the scoring kernel
  const int t0 = a.tile_start[b];
  const int nt = a.tile_start[b + 1] - t0;
  constexpr int per = SEL_LDS_PAIRS / TILE_MAX_PER_SEQ;  // pairs of a tile kept in LDS
  static_assert(per == 64, "one pair per lane of a wave");
  // candidates of a tile kept in LDS: the head space shared by the tiles (a
  // power of two per tile, at most 512)
  const int lh_sh = min(9, 12 - (nt <= 1 ? 0 : 32 - __clz(nt - 1)));
  const int lh = 1 << lh_sh;
  static_assert(SEL_LDS_HEAD == 1 << 12 && SEL_LDS_HEAD / 32 >= TILE_MAX_PER_SEQ, "list heads of every tile fit");
  const int pu_per_tile = per / 4, hu_per_tile = lh / 2;

  // 1. one batch of loads: every tile's pair count, the head of its (bin,
  //    count) list and the head of its candidate list; the pairs are summed
  //    into an LDS histogram (thread t then holds bins NBINS - 4t - 4 ..
  //    NBINS - 4t - 1: ascending threads walk the bins in descending order)
  static_assert(NBINS == 4 * SEL_THREADS, "one uint4 of the histogram per thread");
  const int hq = SEL_THREADS - 1 - tid;
  reinterpret_cast<uint4*>(shist)[tid] = uint4{0u, 0u, 0u, 0u};
  if (tid < 64) reinterpret_cast<uint4*>(h256)[tid] = uint4{0u, 0u, 0u, 0u};
  constexpr int UP = SEL_LDS_PAIRS / 4 / SEL_THREADS, UH = SEL_LDS_HEAD / 2 / SEL_THREADS;
  uint4 pv[UP], hv[UH];
  uint32_t pnp[UP];
#pragma unroll
  for (int k = 0; k < UP; ++k) {
    const int u = tid + k * SEL_THREADS;
    pnp[k] = 0;
    if (u < nt * pu_per_tile) {
      const int j = u / pu_per_tile, part = u % pu_per_tile;
      pnp[k] = P.tile_meta[t0 + j].y;
      pv[k] = *reinterpret_cast<const uint4*>(P.tile_pairs + (size_t)(t0 + j) * PAIR_CAP + part * 4);
    }
  }
#pragma unroll
  for (int k = 0; k < UH; ++k) {
    const int u = tid + k * SEL_THREADS;
    if (u < nt * hu_per_tile) {
      const int j = u / hu_per_tile, part = u % hu_per_tile;
      hv[k] = *reinterpret_cast<const uint4*>(P.tile_list + (size_t)(t0 + j) * TILE_CAP + part * 2);
    }
  }
  uint32_t my_np = 0;
  if (tid < nt) my_np = P.tile_meta[t0 + tid].y;
  for (int i = tid; i < SEL_BUCKETS; i += SEL_THREADS) bcnt[i] = 0;
  lds_barrier();  // histogram zero (the loads stay in flight)
#pragma unroll
  for (int k = 0; k < UP; ++k) {
    const int u = tid + k * SEL_THREADS;
    if (u < nt * pu_per_tile) {
      const int j = u / pu_per_tile, part = u % pu_per_tile;
      const uint32_t w[4] = {pv[k].x, pv[k].y, pv[k].z, pv[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (part * 4 + e < (int)pnp[k]) {
          lpairs[j * per + part * 4 + e] = w[e];
          atomicAdd(&shist[w[e] >> 16], w[e] & 0xFFFFu);
        }
    }
  }
#pragma unroll
  for (int k = 0; k < UH; ++k) {
    const int u = tid + k * SEL_THREADS;
    if (u < nt * hu_per_tile) {
      const int j = u / hu_per_tile, part = u % hu_per_tile;
      lhead[j * lh + part * 2] = ((uint64_t)hv[k].y << 32) | hv[k].x;
      lhead[j * lh + part * 2 + 1] = ((uint64_t)hv[k].w << 32) | hv[k].z;
    }
  }
  // The offsets of the pairs beyond a tile's LDS slice (rare: a tile spread
  // over more than `per` bins), which are read from global memory as one flat
  // range over tiles.
  const uint32_t o = (tid < nt && my_np > (uint32_t)per) ? my_np - per : 0u;
  if (tid < nt) npr[tid] = my_np;
  if (nt <= 64 && wave == 0) {
    uint32_t tot;
    const uint32_t e = wave_exclusive_scan(o, &tot);
    if (tid < nt) ovf_off[tid] = e;
    if (tid == 0) ovf_off[nt] = tot;
  }
  __syncthreads();  // pairs, list heads and offsets published
  if (nt > 64) {    // uniform: more tiles than one wave scans
    uint32_t tot;
    const uint32_t e = block_exclusive_scan(o, scr + NWV, &tot);
    if (tid < nt) ovf_off[tid] = e;
    if (tid == 0) ovf_off[nt] = tot;
    __syncthreads();
  }
  const uint32_t novf = ovf_off[nt];
  if (novf) {  // uniform: the pairs past the LDS slices enter the histogram too
    for (uint32_t i = tid; i < novf; i += SEL_THREADS) {
      const int j = owner_of(ovf_off, nt, i);
      const uint32_t w = P.tile_pairs[(size_t)(t0 + j) * PAIR_CAP + per + (i - ovf_off[j])];
      atomicAdd(&shist[w >> 16], w & 0xFFFFu);
    }
    lds_barrier();
  }
  // suffix counts of the histogram by wave
  const uint4 hcnt = reinterpret_cast<const uint4*>(shist)[hq];
  const uint32_t local = hcnt.x + hcnt.y + hcnt.z + hcnt.w;
  const uint32_t xin = wave_inclusive_scan(local);
  if (lane == 63) scr[wave] = xin;
  lds_barrier();
  // the boundary: the highest bin whose suffix count reaches k
  int bstar;
  uint32_t n_gt, total = 0, above = xin - local;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const uint32_t t_ = scr[w];
    total += t_;
    if (w < wave) above += t_;
  }
  if (tid == 0 && total < K) {
    scr[SCR_RES] = 0xFFFFFFFFu;
    scr[SCR_RES + 1] = total;
  }
  if (total >= K && above < K && above + local >= K) {
    const uint32_t c4[4] = {hcnt.w, hcnt.z, hcnt.y, hcnt.x};
    uint32_t run = above;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run + c4[j] >= K) {
        scr[SCR_RES] = (uint32_t)(4 * hq + 3 - j);
        scr[SCR_RES + 1] = run;
        break;
      }
      run += c4[j];
    }
  }
  __syncthreads();
  bstar = (int)scr[SCR_RES];
  n_gt = scr[SCR_RES + 1];
  // bstar >= 0: the tiles together kept at least k candidates.
  const uint32_t m = K - n_gt;
  // 2. per tile: candidates above the boundary bin and in it, one wave per
  //    tile, a lane per LDS pair (a tile's pairs cover distinct bins; at most
  //    one is the boundary's), summed across the wave
  for (int j = wave; j < nt; j += NWV) {
    const bool v = (uint32_t)lane < npr[j];
    const uint32_t w = v ? lpairs[j * per + lane] : 0u;
    const int bin = (int)(w >> 16);
    const uint32_t g_ = wave_inclusive_scan(v && bin > bstar ? w & 0xFFFFu : 0u);
    const uint32_t d_ = wave_inclusive_scan(v && bin == bstar ? w & 0xFFFFu : 0u);
    if (lane == 63) {
      ngt[j] = g_;
      nbd[j] = d_;
    }
  }
  __syncthreads();
  for (uint32_t i = tid; i < novf; i += SEL_THREADS) {
    const int j = owner_of(ovf_off, nt, i);
    const uint32_t w = P.tile_pairs[(size_t)(t0 + j) * PAIR_CAP + per + (i - ovf_off[j])];
    const int bin = (int)(w >> 16);
    if (bin > bstar) atomicAdd(&ngt[j], w & 0xFFFFu);
    else if (bin == bstar) nbd[j] = w & 0xFFFFu;
  }
  if (novf) __syncthreads();  // uniform
  // offsets of each tile's candidates in the selection and the boundary list
  if (nt <= 64) {  // uniform: one wave scans the tiles
    if (wave == 0) {
      const uint32_t g_ = tid < nt ? ngt[tid] : 0u, d_ = tid < nt ? nbd[tid] : 0u;
      uint32_t tg, tb;
      const uint32_t eg = wave_exclusive_scan(g_, &tg);
      const uint32_t eb = wave_exclusive_scan(d_, &tb);
      if (tid < nt) {
        sure_off[tid] = eg;
        bnd_off[tid] = eb;
      }
      if (tid == 0) {
        sure_off[nt] = tg;
        bnd_off[nt] = tb;
      }
    }
  } else {
    const uint32_t g_ = tid < nt ? ngt[tid] : 0u, d_ = tid < nt ? nbd[tid] : 0u;
    uint32_t tg, tb;
    const uint32_t eg = block_exclusive_scan(g_, scr, &tg);
    const uint32_t eb = block_exclusive_scan(d_, scr, &tb);
    if (tid < nt) {
      sure_off[tid] = eg;
      bnd_off[tid] = eb;
    }
    if (tid == 0) {
      sure_off[nt] = tg;
      bnd_off[nt] = tb;
    }
  }
  __syncthreads();
  // 3. candidates: one wave per tile copies the tile's entries above the
  //    boundary bin to the selection and its boundary-bin entries (as
  //    (score, -id) keys) to the boundary list (both are prefixes of the
  //    tile's bin-ordered list, read from its LDS head where possible)
  const uint32_t nbnd = bnd_off[nt];
  // the sequence's candidate lists as a buffer resource: a global load the
  // compiler cannot merge with the LDS read into one flat access
  const auto lists = __builtin_amdgcn_make_buffer_rsrc(P.tile_list + (size_t)t0 * TILE_CAP, 0,
                                                       nt * TILE_CAP * 8, 0x00020000);
  auto entry = [&](int j, uint32_t e) -> uint64_t {  // e-th candidate of tile j
    if (e < (uint32_t)lh) return lhead[j * lh + e];
    const v2u w = __builtin_amdgcn_raw_buffer_load_b64(lists, (j * TILE_CAP + (int)e) * 8, 0, 0);
    return ((uint64_t)w.y << 32) | w.x;
  };
  const bool in_lds = nbnd <= SEL_CAND;
  // one wave per tile, a lane per entry (entries past the tile's LDS head come
  // from global memory)
  for (int j = wave; j < nt; j += NWV) {
    const uint32_t gj = ngt[j], nj = gj + (in_lds ? nbd[j] : 0u);
    const uint32_t so = sure_off[j], bo = bnd_off[j];
#pragma unroll 2
    for (uint32_t e = lane; e < nj; e += 64) {
      const uint64_t ent = entry(j, e);
      if (e < gj) sel[so + e] = (uint32_t)ent;
      else cand[bo + (e - gj)] = rank_key(key_score(ent), (uint32_t)ent);
    }
  }
  if (tid == 0 && in_lds && (nbnd & 1)) cand[nbnd] = 0;  // pad to an even count for paired reads (ranks below all)
  const uint32_t nsure = sure_off[nt];
  auto bnd_key = [&](uint32_t i) -> uint64_t {
    const int j = owner_of(bnd_off, nt, i);
    const uint64_t e = entry(j, ngt[j] + (i - bnd_off[j]));
    return rank_key(key_score(e), (uint32_t)e);
  };
  __syncthreads();
  // 4. the m best boundary candidates
  if (in_lds) {
    const uint64_t* rk = cand;  // keys to rank, how many, how many to take, where they go
    uint32_t nr = nbnd, mr = m, out0 = nsure;
    if (nbnd > (uint32_t)SEL_REFINE) {  // uniform
      // one more histogram level on the 8 score bits below the boundary bin's
      // resolution (inside a bin every score shares the bits above them, so
      // the level is monotone in the score; a bin below 64 holds one score and
      // one sub-bin): entries of higher sub-bins are selected outright, the
      // sub-boundary's go to a short list that is ranked in full
      const int sh = bstar < 64 ? 0 : max((bstar >> 6) + 5 - 14, 0);
      for (uint32_t i = tid; i < nbnd; i += SEL_THREADS) atomicAdd(&h256[(key_score(cand[i]) >> sh) & 255u], 1u);
      lds_barrier();
      if (wave == 0) {  // lane l holds sub-bins 4(63 - l) .. +3: ascending lanes walk down
        const uint4 c = reinterpret_cast<const uint4*>(h256)[63 - lane];
        const uint32_t loc = c.x + c.y + c.z + c.w;
        const uint32_t above = wave_inclusive_scan(loc) - loc;
        if (above < m && above + loc >= m) {
          const uint32_t c4[4] = {c.w, c.z, c.y, c.x};
          uint32_t run = above;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (run + c4[j] >= m) {
              scr[SCR_RES + 5] = (uint32_t)(4 * (63 - lane) + 3 - j);
              scr[SCR_RES + 6] = run;
              break;
            }
            run += c4[j];
          }
        }
        if (lane == 0) {
          scr[SCR_RES + 7] = 0;  // append cursors: outright, sub-boundary
          scr[SCR_RES + 8] = 0;
        }
      }
      lds_barrier();
      const uint32_t sb = scr[SCR_RES + 5], n_above = scr[SCR_RES + 6];
      uint64_t* sub = reinterpret_cast<uint64_t*>(lpairs);  // the pairs are dead by now
      static_assert(SEL_LDS_PAIRS * 4 >= (SEL_CAND + 2) * 8, "sub-boundary list fits in the pair space");
      for (uint32_t i = tid - lane; i < nbnd; i += SEL_THREADS) {  // whole waves (ballots)
        const bool v = i + lane < nbnd;
        const uint64_t key = v ? cand[i + lane] : 0ull;
        const uint32_t sk = (key_score(key) >> sh) & 255u;
        const uint32_t ph = wave_append(v && sk > sb, &scr[SCR_RES + 7]);
        const uint32_t pe = wave_append(v && sk == sb, &scr[SCR_RES + 8]);
        if (v && sk > sb) sel[nsure + ph] = key_id(key);
        else if (v && sk == sb) sub[pe] = key;
      }
      lds_barrier();
      nr = scr[SCR_RES + 8];
      if (tid == 0 && (nr & 1)) sub[nr] = 0;  // even count for paired reads (ranks below all)
      lds_barrier();
      rk = sub;
      mr = m - n_above;
      out0 = nsure + n_above;
    }
    // all-pairs rank: T adjacent lanes per key (T = 1 .. 64, the most that
    // keeps every key in one pass when there are few), each counting over
    // every T-th pair of keys, summed across the T lanes
    const uint32_t npair = (nr + 1) / 2;
    const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(rk);
    int T = 1;
    while (T < 64 && nr * (uint32_t)T * 2 <= (uint32_t)SEL_THREADS) T *= 2;
    const int per_pass = SEL_THREADS / T;
    for (uint32_t base = 0; base < nr; base += per_pass) {  // uniform
      const uint32_t i = base + tid / T;
      const int part = tid % T;
      uint32_t rank = 0;
      uint64_t ki = 0;
      if (i < nr) {
        ki = rk[i];
#pragma unroll 4
        for (uint32_t j = part; j < npair; j += T) {
          const ulonglong2 v = c2[j];
          rank += (v.x > ki) + (v.y > ki);
        }
      }
      for (int o = 1; o < T; o <<= 1) rank += __shfl_xor(rank, o, 64);
      if (i < nr && part == 0 && rank < mr) sel[out0 + rank] = key_id(ki);
    }
  } else {
    const uint64_t thr = radix_select_threshold(
        [&](auto f) {
          for (uint32_t i = tid; i < nbnd; i += SEL_THREADS) f(bnd_key(i));
        },
        m, h256, scr);
    if (tid == 0) scr[SCR_RES + 9] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < nbnd; i += SEL_THREADS) {
      const uint64_t key = bnd_key(i);
      if (key >= thr) {
        const uint32_t p = nsure + atomicAdd(&scr[SCR_RES + 9], 1u);
        if (p < MAX_K) sel[p] = key_id(key);
      }
    }
  }
  __syncthreads();
  // ascending order: counting sort on the high bits of the id (buckets of
  // 2^sh groups, at most SEL_BUCKETS of them, zeroed at the start), then a
  // rank inside the bucket
  int sh = 0;
  while ((G - 1) >> sh >= SEL_BUCKETS) ++sh;
  const bool mine = tid < (int)K;
  const uint32_t v = mine ? sel[tid] : 0u;
  const int bk = (int)(v >> sh);
  if (mine) atomicAdd(&bcnt[bk], 1u);
  __syncthreads();
  {
    static_assert(SEL_BUCKETS == 2 * SEL_THREADS, "two buckets per thread");
    const uint32_t c0 = bcnt[2 * tid], c1 = bcnt[2 * tid + 1], cs = c0 + c1;
    const uint32_t x = wave_inclusive_scan(cs);
    if (lane == 63) scr[wave] = x;
    __syncthreads();
    uint32_t e = x - cs;
#pragma unroll
    for (int w = 0; w < NWV; ++w)
      if (w < wave) e += scr[w];
    bbase[2 * tid] = e;
    bbase[2 * tid + 1] = e + c0;
    bcnt[2 * tid] = 0;  // reused as the fill cursor
    bcnt[2 * tid + 1] = 0;
  }
  __syncthreads();
  if (mine) bstage[bbase[bk] + atomicAdd(&bcnt[bk], 1u)] = v;
  __syncthreads();
  int32_t* orow = P.out_idx + (size_t)b * K;
  if (mine) {
    const uint32_t b0 = bbase[bk], n = bcnt[bk];
    uint32_t rank = 0;
    for (uint32_t j = 0; j < n; ++j) rank += bstage[b0 + j] < v;
    orow[b0 + rank] = (int32_t)v;
  }
  if (tid == 0) P.out_count[b] = (int32_t)K;
}

isa_status launch_indexer_decode(const BatchArgs& a, const int8_t* q, const int8_t* hw, const int8_t* pooled,
                                 const int32_t* bt, const DecodeWs& w, int32_t* out_idx, int32_t* out_count,
                                 int32_t* scores_out, int32_t ld_scores, hipStream_t stream) {
  DecodePtrs P{q, hw, pooled, bt, w.tile_meta, w.tile_pairs, w.tile_list, out_idx, out_count,
               scores_out, ld_scores, w.err};
  const int ntiles = a.tile_start[a.batch];
  if (launch_timed(ISA_TIMER_INDEXER_SCORE, k_indexer_score, dim3(ntiles), dim3(DEC_THREADS), stream, a, P) !=
      hipSuccess)
    return ISA_ERR_HIP;
  bool any_sparse = false;
  for (int b = 0; b < a.batch; ++b) any_sparse |= (a.lens[b] + GROUP - 1) / GROUP > a.k;
  if (any_sparse) {
    hipLaunchKernelGGL(k_indexer_select, dim3(a.batch), dim3(SEL_THREADS), 0, stream, a, P);
    if (hipGetLastError() != hipSuccess) return ISA_ERR_HIP;
  }
  return ISA_OK;
}

}  // namespace isa
