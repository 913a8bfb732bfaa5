// indexer_decode.hip -- decode-time lightning-indexer scoring fused with exact
// top-k group selection, for gfx950.
//
// Method (pages cited by title): "GLM-5.3 Sparse Attention은 연산량을 줄이지만 HBM
// 수요는 지속된다" (remio.ai), section "GLM-5.3 Sparse Attention이 실제로 바꾸는 것":
// the indexer scores every earlier position and keeps the top-k; below the
// budget attention stays dense.  "GLM-5.3-Flash vs Qwen3.8-Flash-Next" (alltoptrend),
// section "수렴점 2 — 4배 압축 후 2,048 토큰만 유지": a 32-head indexer over keys pooled
// 4 -> 1, top 512 blocks of 4 tokens.  Score of a pooled group (the pages print
// no formula; this library's contract): S = sum_h w_h * max(0, q_h . k).
//
// Design.  One launch.  The grid is a list of work tiles of 2048 pooled groups
// (32 pages) per sequence.  Each 256-thread workgroup streams its tile's int8
// keys straight from HBM into MFMA operands: v_mfma_i32_32x32x32_i8 with the 32
// indexer heads as M (query in registers, loaded once) and 32 groups as N, four
// MFMAs over the 128 channels; each lane loads 64 contiguous bytes of one key.
// The epilogue applies ReLU and the head weights exactly (u32 multiply-add;
// every partial stays below 2^32) and reduces the heads across the two lane
// halves.  Scores go to LDS (and, optionally, to a checking buffer).
// The workgroup then emits the candidates that can still be in the global
// top-k: it histograms its scores by an 11-bit monotone key, finds the bin
// holding its own k-th best, and writes every candidate from that bin up to a
// per-tile list ordered by bin (descending), and adds those bins to a global
// per-sequence histogram.  The last workgroup of a sequence (atomic ticket)
// finds the global boundary bin, takes the candidates above it, resolves the
// boundary bin exactly by radix select on (score, -id) keys, sorts the k ids
// ascending and writes them; it then clears the histogram and ticket for the
// next call.
#include "isa_launch.hpp"
#include "select_device.hpp"

namespace isa {

constexpr int DEC_THREADS = 256;
constexpr int DEC_STEPS = TILE_G / 128;        // 4 waves x 32 groups per step
constexpr int CAND_LDS = 1024;                 // boundary candidates resolved in LDS

struct DecodePtrs {
  const int8_t* q;
  const int8_t* hw;
  const int8_t* pooled;
  const int32_t* bt;
  uint32_t* ghist;      // [B][NBINS], zero between calls
  uint32_t* tickets;    // [B], zero between calls
  uint32_t* tile_cnt;   // [ntiles]
  uint64_t* tile_list;  // [ntiles][TILE_G]
  int32_t* out_idx;     // [B][k]
  int32_t* out_count;   // [B]
  int32_t* scores_out;  // [B][ld] or null
  int32_t ld_scores;
  uint32_t* err;
};

__device__ __forceinline__ void load_key_operand(v4i (&kb)[4], const int8_t* __restrict__ p) {
  const v4i* v = reinterpret_cast<const v4i*>(p);
  kb[0] = __builtin_nontemporal_load(v + 0);
  kb[1] = __builtin_nontemporal_load(v + 1);
  kb[2] = __builtin_nontemporal_load(v + 2);
  kb[3] = __builtin_nontemporal_load(v + 3);
}

__global__ __launch_bounds__(DEC_THREADS) void k_indexer_decode(const BatchArgs a, const DecodePtrs P) {
  __shared__ uint32_t sc[TILE_G];          // tile scores; later: boundary candidates (as u64)
  __shared__ uint32_t hist[NBINS];         // tile histogram -> emission cursors -> global histogram
  __shared__ uint32_t sel[MAX_K];          // final selection
  __shared__ uint32_t toff[2 * (TILE_MAX_PER_SEQ + 1)];  // per-tile prefix of sure / boundary counts
  __shared__ uint32_t h256[256];
  __shared__ uint32_t scr[SCR_WORDS];
  __shared__ int32_t pages[TILE_G / PAGE_GRP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int b = tile_owner(a, tile);
  const int t0 = a.tile_start[b];
  const int ntiles = a.tile_start[b + 1] - t0;
  const int L = a.lens[b];
  const int G = (L + GROUP - 1) / GROUP;
  const uint32_t K = (uint32_t)a.k;
  const int g0 = (tile - t0) * TILE_G;
  const int gN = min(G - g0, TILE_G);
  const bool dense = G <= (int)K;

  if (dense && P.scores_out == nullptr) {  // fewer than k groups: select them all
    for (int i = tid; i < (int)K; i += DEC_THREADS) P.out_idx[(size_t)b * K + i] = i < G ? i : -1;
    if (tid == 0) P.out_count[b] = G;
    return;
  }

  for (int i = tid; i < NBINS; i += DEC_THREADS) hist[i] = 0;
  if (tid < TILE_G / PAGE_GRP) {
    int j = (g0 / PAGE_GRP) + tid;
    pages[tid] = (tid * PAGE_GRP < gN) ? phys_page(P.bt, a.max_pages, a.num_pages, b, j, P.err) : -1;
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

  // ---- stream the tile: 16 steps of 128 groups (32 per wave) ----
  const int8_t* kbase = P.pooled + (lane >> 5) * 64;
  auto key_ptr = [&](int step) -> const int8_t* {
    int gl = step * 128 + wave * 32 + (lane & 31);
    int pg = pages[gl / PAGE_GRP];
    if (gl >= gN || pg < 0) return nullptr;
    return kbase + ((size_t)pg * PAGE_GRP + (gl % PAGE_GRP)) * IDX_DIM;
  };
  v4i cur[4], nxt[4];
  {
    const int8_t* p = key_ptr(0);
    if (p) load_key_operand(cur, p);
    else cur[0] = cur[1] = cur[2] = cur[3] = v4i{0, 0, 0, 0};
  }
  bool overflow = false;
#pragma unroll 2
  for (int step = 0; step < DEC_STEPS; ++step) {
    if (step + 1 < DEC_STEPS) {
      const int8_t* p = key_ptr(step + 1);
      if (p) load_key_operand(nxt, p);
      else nxt[0] = nxt[1] = nxt[2] = nxt[3] = v4i{0, 0, 0, 0};
    }
    v16i acc = {0};
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[0], cur[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[1], cur[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[2], cur[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[3], cur[3], acc, 0, 0, 0);
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += wv[i] * (uint32_t)max(acc[i], 0);  // ReLU <= 2,064,512 < 2^24
    s += __shfl_xor(s, 32, 64);
    const int gl = step * 128 + wave * 32 + (lane & 31);
    if (lane < 32) {
      bool valid = gl < gN;
      sc[gl] = valid ? s : INVALID_SCORE;
      overflow |= valid && s > 0x7FFFFFFFu;
      if (P.scores_out && valid) P.scores_out[(size_t)b * P.ld_scores + g0 + gl] = (int32_t)s;
    }
    cur[0] = nxt[0];
    cur[1] = nxt[1];
    cur[2] = nxt[2];
    cur[3] = nxt[3];
  }
  if (__any(overflow) && lane == 0) report(P.err, ISA_DERR_SCORE_OVERFLOW);
  __syncthreads();

  if (dense) {  // only reached when scores were requested
    for (int i = tid; i < (int)K; i += DEC_THREADS) P.out_idx[(size_t)b * K + i] = i < G ? i : -1;
    if (tid == 0) P.out_count[b] = G;
    return;
  }

  // ---- local candidates: every score in a bin >= the bin of this tile's k-th best ----
  constexpr int PER = TILE_G / DEC_THREADS;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    uint32_t s = sc[tid + j * DEC_THREADS];
    if (s != INVALID_SCORE) atomicAdd(&hist[score_bin(s)], 1u);
  }
  __syncthreads();
  int bt_local;
  uint32_t n_gt_local, n_valid;
  find_boundary(hist, K, &bt_local, &n_gt_local, &n_valid, scr);
  const int blo = bt_local < 0 ? 0 : bt_local;  // emit all when at most k are valid
  {
    // convert counts of bins >= blo into emission cursors (descending bins), and
    // add them to the sequence's global histogram
    const int per = NBINS / DEC_THREADS;
    const int hi = NBINS - tid * per;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j) {
      int bin = hi - 1 - j;
      if (bin >= blo) local += hist[bin];
    }
    uint32_t tot;
    uint32_t run = block_exclusive_scan(local, scr, &tot);
    for (int j = 0; j < per; ++j) {
      int bin = hi - 1 - j;
      if (bin < blo) break;
      uint32_t c = hist[bin];
      if (c) atomicAdd(&P.ghist[(size_t)b * NBINS + bin], c);
      hist[bin] = run;
      run += c;
    }
    if (tid == 0) P.tile_cnt[tile] = tot;
  }
  __syncthreads();
  uint64_t* list = P.tile_list + (size_t)tile * TILE_G;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int e = tid + j * DEC_THREADS;
    uint32_t s = sc[e];
    if (s == INVALID_SCORE) continue;
    int bin = score_bin(s);
    if (bin < blo) continue;
    uint32_t slot = atomicAdd(&hist[bin], 1u);
    list[slot] = ((uint64_t)s << 32) | (uint32_t)(g0 + e);
  }

  // ---- ticket: the last tile of the sequence finishes the selection ----
  __threadfence();
  __syncthreads();
  if (tid == 0) scr[SCR_RES + 8] = atomicAdd(&P.tickets[b], 1u);
  __syncthreads();
  if ((int)scr[SCR_RES + 8] != ntiles - 1) return;
  __threadfence();

  uint32_t* gh = P.ghist + (size_t)b * NBINS;
  for (int i = tid; i < NBINS; i += DEC_THREADS) {
    hist[i] = __hip_atomic_load(&gh[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&gh[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid == 0) __hip_atomic_store(&P.tickets[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int bstar;
  uint32_t n_gt, total;
  find_boundary(hist, K, &bstar, &n_gt, &total, scr);
  // bstar >= 0 here: the tiles together emitted at least k candidates.
  const uint32_t m = K - n_gt;

  // per tile: [0, ngt_j) above bstar, [ngt_j, nge_j) in bstar (lists are bin-descending)
  uint32_t* sure_off = toff;                          // [ntiles + 1]
  uint32_t* bnd_off = toff + (TILE_MAX_PER_SEQ + 1);  // [ntiles + 1]
  {
    constexpr int PT = (TILE_MAX_PER_SEQ + DEC_THREADS - 1) / DEC_THREADS;
    uint32_t ngt[PT], nbd[PT];
    uint32_t my_gt = 0, my_bd = 0;
#pragma unroll
    for (int r = 0; r < PT; ++r) {
      int j = tid * PT + r;
      ngt[r] = nbd[r] = 0;
      if (j < ntiles) {
        const uint64_t* lj = P.tile_list + (size_t)(t0 + j) * TILE_G;
        uint32_t cnt = P.tile_cnt[t0 + j];
        // first position whose bin <= bstar, then first whose bin < bstar
        uint32_t lo = 0, hi2 = cnt;
        while (lo < hi2) {
          uint32_t mid = (lo + hi2) >> 1;
          if (score_bin(key_score(lj[mid])) > bstar) lo = mid + 1; else hi2 = mid;
        }
        uint32_t a0 = lo;
        hi2 = cnt;
        while (lo < hi2) {
          uint32_t mid = (lo + hi2) >> 1;
          if (score_bin(key_score(lj[mid])) >= bstar) lo = mid + 1; else hi2 = mid;
        }
        ngt[r] = a0;
        nbd[r] = lo - a0;
      }
      my_gt += ngt[r];
      my_bd += nbd[r];
    }
    uint32_t tg, tb;
    uint32_t eg = block_exclusive_scan(my_gt, scr, &tg);
    uint32_t eb = block_exclusive_scan(my_bd, scr, &tb);
#pragma unroll
    for (int r = 0; r < PT; ++r) {
      int j = tid * PT + r;
      if (j < ntiles) {
        sure_off[j] = eg;
        bnd_off[j] = eb;
      }
      eg += ngt[r];
      eb += nbd[r];
    }
    if (tid == 0) {
      sure_off[ntiles] = tg;
      bnd_off[ntiles] = tb;
    }
  }
  __syncthreads();
  const uint32_t nsure = sure_off[ntiles];
  const uint32_t nbnd = bnd_off[ntiles];
  auto owner = [&](const uint32_t* off, uint32_t i) -> int {  // tile j with off[j] <= i < off[j+1]
    int lo = 0, hi2 = ntiles - 1;
    while (lo < hi2) {
      int mid = (lo + hi2 + 1) >> 1;
      if (off[mid] <= i) lo = mid; else hi2 = mid - 1;
    }
    return lo;
  };
  // sure candidates -> sel[0, nsure)
  for (uint32_t i = tid; i < nsure && i < MAX_K; i += DEC_THREADS) {
    int j = owner(sure_off, i);
    sel[i] = (uint32_t)P.tile_list[(size_t)(t0 + j) * TILE_G + (i - sure_off[j])];
  }
  // boundary candidates
  auto bnd_key = [&](uint32_t i) -> uint64_t {
    int j = owner(bnd_off, i);
    // position inside tile j: after its sure part
    uint32_t ngt_j = sure_off[j + 1] - sure_off[j];
    uint64_t e = P.tile_list[(size_t)(t0 + j) * TILE_G + ngt_j + (i - bnd_off[j])];
    return rank_key(key_score(e), (uint32_t)e);
  };
  uint64_t* cand = reinterpret_cast<uint64_t*>(sc);  // TILE_G words = CAND_LDS u64
  const bool in_lds = nbnd <= CAND_LDS;
  if (in_lds)
    for (uint32_t i = tid; i < nbnd; i += DEC_THREADS) cand[i] = bnd_key(i);
  __syncthreads();
  uint64_t thr;
  if (in_lds) {
    thr = radix_select_threshold(
        [&](auto f) {
          for (uint32_t i = tid; i < nbnd; i += DEC_THREADS) f(cand[i]);
        },
        m, h256, scr);
  } else {
    thr = radix_select_threshold(
        [&](auto f) {
          for (uint32_t i = tid; i < nbnd; i += DEC_THREADS) f(bnd_key(i));
        },
        m, h256, scr);
  }
  if (tid == 0) scr[SCR_RES + 9] = 0;
  __syncthreads();
  for (uint32_t i = tid; i < nbnd; i += DEC_THREADS) {
    uint64_t key = in_lds ? cand[i] : bnd_key(i);
    if (key >= thr) {
      uint32_t p = nsure + atomicAdd(&scr[SCR_RES + 9], 1u);
      if (p < MAX_K) sel[p] = key_id(key);
    }
  }
  __syncthreads();
  write_sorted_row(sel, (int)K, (int)K, P.out_idx + (size_t)b * K, P.out_count + b);
}

isa_status launch_indexer_decode(const BatchArgs& a, const int8_t* q, const int8_t* hw, const int8_t* pooled,
                                 const int32_t* bt, const DecodeWs& w, int32_t* out_idx, int32_t* out_count,
                                 int32_t* scores_out, int32_t ld_scores, hipStream_t stream) {
  DecodePtrs P{q, hw, pooled, bt, w.ghist, w.tickets, w.tile_cnt, w.tile_list, out_idx, out_count,
               scores_out, ld_scores, w.err};
  int ntiles = a.tile_start[a.batch];
  hipLaunchKernelGGL(k_indexer_decode, dim3(ntiles), dim3(DEC_THREADS), 0, stream, a, P);
  return hipGetLastError() == hipSuccess ? ISA_OK : ISA_ERR_HIP;
}

}  // namespace isa
