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
// Design.  A workgroup is (query row, token split) with eight waves, and every
// byte of a latent tile is loaded by exactly one of them: wave (cg, th) owns
// latent channels 128cg..128cg+127 and tokens 16th..16th+15 of each 32-token
// tile.  (A layout where several waves load the same rows -- one per block of
// heads -- is capped near 2.3 TB/s of unique bytes by the vector memory path;
// without replication the same gather reaches about 6 TB/s.)  Per tile:
//  * Partial scores S^T = C Q^T over the wave's 128 channels for its 16 tokens
//    and all 64 heads (v_mfma_f32_16x16x32_bf16, tokens = M, heads = N, the
//    query block in registers).  Each lane loads 16 contiguous bytes of a
//    latent row per K step straight from HBM, two tiles ahead.
//  * The same registers, converted to fp16 (exact for bf16 values in the fp16
//    normal range), are stored token-major in LDS as V; the P.V product reads
//    them back transposed (ds_read_b64_tr_b16).  The partial scores go to LDS
//    too.  Operands are not masked: an invisible token's score is discarded
//    by the softmax and its V row is overwritten with zeros.
//  * Wave w owns the softmax of heads 8w..8w+7: it sums the four channel
//    groups' partials for its heads over the 32 tokens, keeps the running
//    reference and sum (base 2; the reference moves only when a head's scores
//    exceed it by more than 8, so p <= 256 and the output rescale is rare) and
//    writes P to LDS as two fp16 terms, p_hi = fp16(p) and p_lo = fp16(p - p_hi),
//    which together carry p to about 2^-22 relative.
//  * Every wave then accumulates O[64 heads x its 64 channels] += P V^T with
//    v_mfma_f32_16x16x32_f16 (heads = M, channels = N, the 32 tokens = K) for
//    p_hi, and once more for p_lo when the tile holds a latent value of at
//    least PV_LO_MIN in magnitude: fp16 probabilities alone would be off by
//    2^-11 of the largest value (at most 2^-8 below that bound), the pair keeps
//    the weighted sum accurate to fp32 accumulation.  The decision is one
//    flag per tile in LDS: with bf16 rows the loading waves raise it from the
//    magnitudes they see while converting (a three-way maximum per word, on
//    the conversion's fp32 intermediates), before the first barrier, so the
//    owners also skip p_lo when it is not needed; with FP8 rows the owners
//    raise it from the row scales.
// Two workgroup barriers per tile, both LDS-only; V is double-buffered.
// A launch of at most 128 (row, split) units runs two workgroups per unit,
// each with 32 of the heads (the same tile loads, half the MFMA and softmax
// work), so that it fills the chip.
// With one split the workgroup normalises and writes the output; otherwise it
// writes its normalised partial O / l with the reference and sum in fp32, and
// k_mla_combine merges the splits by log-sum-exp weights.  The partial is held
// in fp16 when every value of the workgroup's partial is below PART_F16_MAX in
// magnitude (fp16 rounding then moves a value by at most 2^-8), otherwise in
// fp32; the format is recorded per (split, head) beside the reference and sum.
#include <type_traits>

#include "isa_launch.hpp"

namespace isa {

constexpr int MLA_THREADS = 512;  // 8 waves: 4 channel groups x 2 token halves
constexpr int CG_DIM = LAT_DIM / 4;   // channels of a wave's score share (its channel group)
constexpr int KSTEPS = CG_DIM / 32;   // K steps of the score product per wave
constexpr int HBLK = ATT_HEADS / 16;  // 16-head blocks
constexpr int OUT_DIM = LAT_DIM / 8;  // output channels per wave
constexpr int NBLK = OUT_DIM / 16;    // 16-channel blocks of the output per wave
constexpr int OWN_HEADS = ATT_HEADS / 8;  // heads whose softmax a wave owns
constexpr float RESCALE_LOG2 = 8.f;
constexpr int TILE_TOK = 32;
constexpr int V_STRIDE = LAT_DIM + 16;  // halves per V row in LDS (1 KiB + 32 B: rows 8 banks apart)
constexpr int P_STRIDE = 40;   // halves per P row (32 tokens + 8 pad, 80 B)
constexpr int SP_LANES = 96;   // partial-score slots per (half, group, head block): 64 lanes + 8 pad per 16
constexpr int MAX_GPS = MAX_K; // groups per split held in LDS
constexpr int BT_LDS = 1024;   // block-table entries of a row staged in LDS (sequences up to 256K tokens;
                               // for longer rows staging costs more than the round trip it saves)
constexpr int MAX_SPLITS = 32;
constexpr float PART_F16_MAX = 16.f;  // partials below this magnitude are held in fp16
constexpr float PV_LO_MIN = 8.f;      // a tile with a latent value this large takes the p_lo pass
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Two bf16 values (low half first) to two fp16 values.  Exact for values in
// the fp16 normal range, which the latent rows are required to stay in; the
// conversion truncates, which for these values is the same as rounding.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
  return __builtin_bit_cast(uint32_t, h);
}
// The same conversion, also folding both values' magnitudes into mv: one
// three-way maximum with absolute-value source modifiers on the fp32
// intermediates.  Written out, since through fmaxf the compiler would first
// canonicalise each bit-cast operand (one more instruction per value); NaN
// handling does not matter here (a NaN in a visible row makes the output NaN
// whatever is decided).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_mag(uint32_t w, float& mv) {
  const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(mv) : "v"(mv), "v"(lo), "v"(hi));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
// LDS row of token slot t of a tile: slots 8..15 and 24..31 swap their halves,
// so the two 16-lane groups of a transposed read (tokens 8g + 4h + 0..3,
// g = 0, 1) fall on disjoint banks.
__device__ __forceinline__ int vrow(int t) { return t ^ (((t >> 3) & 1) << 2); }
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i%4 of the 8-byte rows addressed by lanes i/4, 4 + i/4,
// 8 + i/4, 12 + i/4.  With lane s addressing token t0 + s/4, channels
// c0 + 4(s%4) .. +3 of a token-major tile, lane i gets channel c0 + i of
// tokens t0 .. t0+3: a quarter of an MFMA operand with tokens as K.
__device__ __forceinline__ v4s lds_read_tr16(const _Float16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)((__attribute__((address_space(3))) _Float16*)p));
}
// slot of a writer lane's partial-score accumulator (8 pad slots per 16 lanes
// keep both the writes and the owners' gathers free of bank conflicts)
__device__ __forceinline__ int sp_slot(int lane) { return lane + 8 * (lane >> 4); }

struct MlaPtrs {
  const uint16_t* q[ISA_MAX_LAYERS];       // per layer sharing the selection
  const void* latent[ISA_MAX_LAYERS];      // bf16 rows, or FP8 E4M3 codes
  const float* lat_scale[ISA_MAX_LAYERS];  // FP8: per-row scales
  float* out[ISA_MAX_LAYERS];
  float* lse[ISA_MAX_LAYERS];              // all null when not requested
  int32_t n_layers;
  int32_t rows;
  const int32_t* bt;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const int32_t* idx;
  const int32_t* count;
  char* o_part;      // [layers][rows][splits][64] slots of 2 KiB: normalised partial O / l of one
                     // head, 512 fp16 (first KiB) or 512 fp32 values
  float* ml_part;    // [layers][rows][splits][64][4]: reference (log2 units), sum, format (1 = fp32), 0
  uint32_t* err;
  int32_t k;
  float c2;  // sm_scale * log2(e)
  int32_t splits;
  int32_t gps;  // groups per split
  int32_t n_units;  // (layer, row, split) units of the launch
  int32_t n_xcd;    // XCDs the launch's workgroups are dispatched over, round-robin
};

// FP8 E4M3 codes of 8 channels to fp16 (exact: every E4M3 value is an fp16
// value), low byte first.
__device__ __forceinline__ v8h fp8x8_to_f16x8(v2i w) {
  typedef _Float16 v2h_ __attribute__((ext_vector_type(2)));
  const v2h_ a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)w.x, 1.0f, false);
  const v2h_ b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)w.x, 1.0f, true);
  const v2h_ c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)w.y, 1.0f, false);
  const v2h_ d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((uint32_t)w.y, 1.0f, true);
  return v8h{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// FP8 selects the cache format: bf16 rows (1 KiB per token), or E4M3 codes
// (512 B per token) with one fp32 scale per row.  The FP8 path decodes the
// codes to fp16 exactly and uses fp16 MFMA for both products, with the query
// converted to fp16 once; a token's scale multiplies its scores and is folded
// into its probability for the P.V product (the normalising sum stays unscaled).
// MULTI: several layers share the selection (the layer is part of the grid);
// a single-layer launch keeps every pointer a static kernel argument.
// NH: heads per workgroup.  With 32, two workgroups share a (row, split) unit,
// one per half of the heads, numbered so that both land on the same XCD (the
// second fetch of a latent row comes from its L2): half the MFMA and softmax
// work per tile, for launches that would otherwise leave CUs idle.
template <bool FP8, bool MULTI, int NH>
__global__ __launch_bounds__(MLA_THREADS) void k_mla_split(const BatchArgs a, const MlaPtrs P) {
  constexpr int HB = NH / 16;            // 16-head blocks of the workgroup
  constexpr int NSW = NH / OWN_HEADS;    // waves that own softmax heads
  using LoadT = typename std::conditional<FP8, v2i, v4i>::type;  // one lane's 8 channels of a row
  using QOpT = typename std::conditional<FP8, v8h, v8bf>::type;
  __shared__ __attribute__((aligned(16))) _Float16 vt[2][TILE_TOK * V_STRIDE];  // 2 x 33 KiB: fp16 V of a tile, double-buffered
  __shared__ v4f sp[2][4][HB][SP_LANES];                  // 48 KiB (64 heads): partial S^T [half][group][head block][lane]
  __shared__ _Float16 pb[NH * P_STRIDE];                  // 5 KiB (64 heads): p_hi of the tile [head][token]
  __shared__ _Float16 pbl[NH * P_STRIDE];                 // 5 KiB (64 heads): p_lo of the tile
  __shared__ __attribute__((aligned(16))) float alpha_s[NH];
  __shared__ __attribute__((aligned(16))) uint32_t flag_s[8];
  __shared__ uint32_t big_s;  // a partial value reached PART_F16_MAX: the split's partial is held in fp32
  __shared__ uint32_t vflag_s[2];  // per V buffer: the tile needs the p_lo pass (a large value or row scale)
  __shared__ float fin_s[2][NH];
  __shared__ __attribute__((aligned(16))) uint32_t trow[MAX_GPS * GROUP];  // latent row of each token slot, ~0 if not visible
  __shared__ int32_t bt_s[BT_LDS];                        // 4 KiB: the row's block-table entries

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = wave & 3, th = wave >> 2;   // channels 128cg.., tokens 16th.. of each tile
  int unit = (int)blockIdx.x, hh = 0;  // (layer, row, split) unit and half of the heads
  if constexpr (NH < ATT_HEADS) {
    const int nx = P.n_xcd;  // dispatch is round-robin over the XCDs
    const int slot = (int)blockIdx.x / nx;
    hh = slot & 1;
    unit = (slot >> 1) * nx + (int)blockIdx.x % nx;
    if (unit >= P.n_units) return;  // the whole workgroup
  }
  const int h0 = hh * NH;  // first head of this workgroup
  const int layer = MULTI ? unit / (P.rows * P.splits) : 0;  // layers sharing the selection
  const int rs = MULTI ? unit % (P.rows * P.splits) : unit;
  const int r = rs / P.splits;
  const int split = rs % P.splits;
  const uint16_t* const q = P.q[layer];
  const char* const latent = static_cast<const char*>(P.latent[layer]);
  const float* const lscale = P.lat_scale[layer];
  constexpr int ROW_BYTES = FP8 ? LAT_DIM : LAT_DIM * 2;
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
  // query operand (B = Q^T), fetched in the same round as the group ids:
  // lane -> head 16hb + lq, channels 128cg + 32c + 8lg .. +7 (bf16 bits; the
  // FP8 path converts it to fp16 once the token table is built).  The two
  // waves of a channel group (token halves th = 0, 1) need the same operand:
  // each loads the head blocks of its half, 16th .. (HB/2 blocks), and takes
  // the other half from its partner through LDS, so that every query byte is
  // read from memory once per workgroup.
  static_assert(HB % 2 == 0, "head blocks split between the two token halves");
  constexpr int QH = HB / 2;
  v4i qmine[QH][KSTEPS];
  {
    const uint16_t* qp = q + ((size_t)r * ATT_HEADS + h0 + 16 * QH * th + lq) * LAT_DIM + cg * CG_DIM + lg * 8;
#pragma unroll
    for (int hh = 0; hh < QH; ++hh)
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) qmine[hh][c] = *reinterpret_cast<const v4i*>(qp + (size_t)hh * 16 * LAT_DIM + c * 32);
  }
  // the row's block-table entries, fetched in the same round as the group ids
  // (one dependent global round trip less before the first latent load)
  const int npg = (L + PAGE_TOK - 1) / PAGE_TOK;
  const bool bt_staged = npg <= BT_LDS;
  if (bt_staged)
    for (int j = tid; j < npg; j += MLA_THREADS) bt_s[j] = P.bt[(size_t)seq * a.max_pages + j];
  if (!seq_ok || pos < 0 || pos >= L || cnt < 0 || cnt > P.k) {
    if (tid == 0) report(P.err, ISA_DERR_ROW_RANGE);
    cnt = 0;
  }
  const int G = (L + GROUP - 1) / GROUP;
  const int jbeg = min(cnt, jbeg0);
  const int jend = min(cnt, jbeg + P.gps);
  const int ng = jend - jbeg;
  if (bt_staged) __syncthreads();  // uniform across the workgroup
  // token table of the split: one block-table lookup per selected group
#pragma unroll
  for (int e = 0; e < MAX_GPS / MLA_THREADS + 1; ++e) {
    const int j = tid + e * MLA_THREADS;
    if (j >= ng) continue;
    const int g = gid[e];
    int pg = -1;
    if (g < 0 || g >= G) {
      report(P.err, ISA_DERR_ROW_RANGE);
    } else if (bt_staged) {
      pg = bt_s[(g * GROUP) / PAGE_TOK];
      if (pg < 0 || pg >= a.num_pages) {
        report(P.err, ISA_DERR_PAGE_OOB);
        pg = -1;
      }
    } else {
      pg = phys_page(P.bt, a.max_pages, a.num_pages, seq, (g * GROUP) / PAGE_TOK, P.err);
    }
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      int tok = g * GROUP + i;
      bool vis = pg >= 0 && tok < L && tok <= pos;
      trow[j * GROUP + i] = vis ? (uint32_t)pg * PAGE_TOK + (uint32_t)(tok % PAGE_TOK) : 0xFFFFFFFFu;
    }
  }
  // softmax state of the owned head h = 8 wave + lane % 8 (identical in the
  // eight lanes of a head; l_run is this lane's share of the sum)
  const int own_h = OWN_HEADS * wave + (lane & 7);
  const int own_tq = lane >> 3;  // tokens 4 own_tq .. +3 of the tile
  if (tid < 8) flag_s[tid] = 0u;  // waves without softmax heads never set theirs
  if (tid == 0) big_s = 0u;
  if (tid < 2) vflag_s[tid] = 0u;
  // this wave's half of the query operand to LDS (the V tiles, free until the
  // first tile): wave w's entries at 1 KiB (QH KSTEPS w + entry), 16 B per lane
  v4i* qx = reinterpret_cast<v4i*>(&vt[0][0]);
  static_assert(MLA_THREADS / 64 * QH * KSTEPS * 1024 <= (int)sizeof(vt), "query exchange fits in the V tiles");
#pragma unroll
  for (int hh = 0; hh < QH; ++hh)
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) qx[((wave * QH + hh) * KSTEPS + c) * 64 + lane] = qmine[hh][c];
  lds_barrier();  // token table complete, query halves published
  v4i qother[QH][KSTEPS];
  {
    const int pw = wave ^ 4;  // the partner: same channel group, other token half
#pragma unroll
    for (int hh = 0; hh < QH; ++hh)
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) qother[hh][c] = qx[((pw * QH + hh) * KSTEPS + c) * 64 + lane];
  }
  lds_barrier();  // every wave has its operand: the V tiles are free again

  const int nslot = ng * GROUP;
  const int ntile = (nslot + TILE_TOK - 1) / TILE_TOK;
  QOpT qop[HB][KSTEPS];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      // head block hb: this wave's own load when it lies in its half
      const v4i w = (hb < QH) == (th == 0) ? qmine[hb % QH][c] : qother[hb % QH][c];
      if constexpr (FP8)
        qop[hb][c] = __builtin_bit_cast(v8h, v4i{(int)bf16x2_to_f16x2((uint32_t)w[0]), (int)bf16x2_to_f16x2((uint32_t)w[1]),
                                                 (int)bf16x2_to_f16x2((uint32_t)w[2]), (int)bf16x2_to_f16x2((uint32_t)w[3])});
      else
        qop[hb][c] = __builtin_bit_cast(v8bf, w);
    }
  v4f o[HB][NBLK];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int nb = 0; nb < NBLK; ++nb) o[hb][nb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;

  // This lane's load of tile t: token 16th + lq, channels 128cg + 8lg + 32c.
  // Loads are unconditional (an invisible token reads row 0 of the pool and is
  // zeroed by its mask), so no branch separates a load from its use and the
  // compiler waits for exactly the loads it consumes.
  auto row_of = [&](int t, int& mask) -> const LoadT* {
    const int slot = t * TILE_TOK + th * 16 + lq;
    const uint32_t tr = trow[min(slot, MAX_GPS * GROUP - 1)];  // always in range; masked below
    const bool vis = t < ntile && slot < nslot && tr != 0xFFFFFFFFu;
    mask = vis ? -1 : 0;
    const uint32_t row = vis ? tr : 0u;
    return reinterpret_cast<const LoadT*>(latent + (size_t)row * ROW_BYTES + (cg * CG_DIM + lg * 8) * (ROW_BYTES / LAT_DIM));
  };
  // FP8: the row scales of the 4 tokens of this lane's softmax group in tile t
  // (row 0's when the group is not visible; masked at use)
  auto scales_of = [&](int t) -> const float4* {
    const int sbase = t * TILE_TOK + 4 * own_tq;
    const uint32_t tr = trow[min(sbase, MAX_GPS * GROUP - 4)];
    const bool vis = t < ntile && sbase < nslot && tr != 0xFFFFFFFFu;
    return reinterpret_cast<const float4*>(lscale + (vis ? tr : 0u));
  };

  // one tile: partial scores, V, softmax of the owned heads, P.V
  auto tile_step = [&](int t, LoadT (&buf)[KSTEPS], int& bmask, float4& sbuf) {
    const int vb = t & 1;
    _Float16* vtb = vt[vb];
    v4f acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = v4f{0.f, 0.f, 0.f, 0.f};
    int nmask;
    const LoadT* nsrc = row_of(t + 2, nmask);
    // Operands unmasked: an invisible token's score is discarded by the
    // softmax (its x is -inf whatever the partials hold), and its V row is
    // overwritten with zeros below, so that P = 0 meets finite values.
    float mv = 0.f;  // bf16: largest magnitude of this lane's V values
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      v4i vh;  // V in fp16, token-major: this lane's 8 channels of token 16th + lq
      if constexpr (FP8) {
        const v8h kh = fp8x8_to_f16x8(buf[c]);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, qop[hb][c], acc[hb], 0, 0, 0);
        vh = __builtin_bit_cast(v4i, kh);
      } else {
        const v4i kv = buf[c];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kv), qop[hb][c], acc[hb], 0, 0, 0);
        vh = v4i{(int)bf16x2_to_f16x2_mag((uint32_t)kv[0], mv), (int)bf16x2_to_f16x2_mag((uint32_t)kv[1], mv),
                 (int)bf16x2_to_f16x2_mag((uint32_t)kv[2], mv), (int)bf16x2_to_f16x2_mag((uint32_t)kv[3], mv)};
      }
      *reinterpret_cast<v4i*>(&vtb[vrow(th * 16 + lq) * V_STRIDE + cg * CG_DIM + c * 32 + lg * 8]) = vh;
      buf[c] = nsrc[c * 4];  // refill with tile t + 2
    }
    if (!bmask) {  // invisible token (rare: a split's tail or positions past the query)
      asm volatile("" ::: "memory");  // keep these stores apart from the ones above
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c)
        *reinterpret_cast<v4i*>(&vtb[vrow(th * 16 + lq) * V_STRIDE + cg * CG_DIM + c * 32 + lg * 8]) = v4i{0, 0, 0, 0};
    }
    // bf16: a visible value of at least PV_LO_MIN in magnitude anywhere in the
    // tile turns on the p_lo pass for the whole workgroup
    if constexpr (!FP8) {
      if (__any(bmask && mv >= PV_LO_MIN) && lane == 0) vflag_s[vb] = 1u;
    }
    bmask = nmask;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) sp[th][cg][hb][sp_slot(lane)] = acc[hb];
    lds_barrier();  // partial scores and V of this tile complete

    // ---- softmax of the owned heads over the tile's 32 tokens ----
    if (wave < NSW) {
      const int hb = own_h >> 4, hl = own_h & 15;
      const int tq = own_tq, th2 = tq >> 2;
      v4f s = sp[th2][0][hb][sp_slot(hl + 16 * (tq & 3))];
#pragma unroll
      for (int g2 = 1; g2 < 4; ++g2) s += sp[th2][g2][hb][sp_slot(hl + 16 * (tq & 3))];
      const int sbase = t * TILE_TOK + 4 * tq;
      const uint4 tr = *reinterpret_cast<const uint4*>(&trow[min(sbase, MAX_GPS * GROUP - 4)]);
      const uint32_t trv[4] = {tr.x, tr.y, tr.z, tr.w};
      float x[4], st[4];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = sbase + i < nslot && trv[i] != 0xFFFFFFFFu;
        if constexpr (FP8) {
          st[i] = vis ? (&sbuf.x)[i] : 0.f;
          x[i] = vis ? s[i] * st[i] * P.c2 : -INFINITY;
        } else {
          x[i] = vis ? s[i] * P.c2 : -INFINITY;
        }
        mt = fmaxf(mt, x[i]);
      }
      const bool moved = __any(mt > m_ref + RESCALE_LOG2);
      float alpha = 1.f;
      if (moved) {  // wave-uniform: move the reference of every owned head to its max so far
        mt = fmaxf(mt, __shfl_xor(mt, 8, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_ref, mt);
        alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        l_run *= alpha;
        m_ref = m_new;
      }
      // every owner publishes its heads' factors (1 when it did not move) and
      // whether it moved, so one rescale pass serves all heads
      if (tq == 0) alpha_s[own_h] = alpha;
      if (lane == 0) flag_s[wave] = moved ? 1u : 0u;
      float ps = 0.f;
      float pw[4];
      v4h ph;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[i] - m_ref);
        ps += pr;
        pw[i] = pr;
        if constexpr (FP8) pw[i] = pr * st[i];  // the row scale enters P.V through P
        ph[i] = (_Float16)pw[i];
      }
      l_run += ps;
      *reinterpret_cast<v4h*>(&pb[own_h * P_STRIDE + 4 * tq]) = ph;
      // p_lo only for a tile that needs it: with bf16 rows the loading waves
      // have flagged a large value before the barrier above; with FP8 rows the
      // owners flag a large row scale here.  The flag of the other V buffer is
      // cleared here: every wave has finished the tile that used it, and none
      // can reach the next one before the barrier below.
      bool lo;
      if constexpr (FP8) {
        lo = __any(!(st[0] * 448.f < PV_LO_MIN) || !(st[1] * 448.f < PV_LO_MIN) || !(st[2] * 448.f < PV_LO_MIN) ||
                   !(st[3] * 448.f < PV_LO_MIN));
        if (lane == 0 && lo) vflag_s[vb] = 1u;
      } else {
        lo = __builtin_amdgcn_readfirstlane(vflag_s[vb]) != 0u;
      }
      if (lane == 0 && wave == 0) vflag_s[vb ^ 1] = 0u;
      if (lo) {
        v4h pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) pl[i] = (_Float16)(pw[i] - (float)ph[i]);  // exact difference, rounded once
        *reinterpret_cast<v4h*>(&pbl[own_h * P_STRIDE + 4 * tq]) = pl;
      }
      if constexpr (FP8) sbuf = *scales_of(t + 2);  // refill with tile t + 2, after the latent rows
    }
    lds_barrier();  // P, reference moves complete

    // ---- O[64 heads x this wave's 64 channels] += P V ----
    const uint4 f0 = *reinterpret_cast<const uint4*>(&flag_s[0]);
    const uint4 f1 = *reinterpret_cast<const uint4*>(&flag_s[4]);
    // the flags are the same in every lane: a scalar branch
    if (__builtin_amdgcn_readfirstlane(f0.x | f0.y | f0.z | f0.w | f1.x | f1.y | f1.z | f1.w) != 0u) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float4 al = *reinterpret_cast<const float4*>(&alpha_s[hb * 16 + 4 * lg]);
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb) {
          o[hb][nb][0] *= al.x;
          o[hb][nb][1] *= al.y;
          o[hb][nb][2] *= al.z;
          o[hb][nb][3] *= al.w;
        }
      }
    }
    // V operand: lane (lq, lg) gets channel 16nb + lq of tokens 8lg .. 8lg+7
    const _Float16* vr0 = &vtb[vrow(8 * lg + (lq >> 2)) * V_STRIDE + wave * OUT_DIM + 4 * (lq & 3)];
    const _Float16* vr1 = &vtb[vrow(8 * lg + 4 + (lq >> 2)) * V_STRIDE + wave * OUT_DIM + 4 * (lq & 3)];
    auto v_op = [&](int nb) -> v8h {
      const v4s v0 = lds_read_tr16(vr0 + nb * 16), v1 = lds_read_tr16(vr1 + nb * 16);
      return __builtin_bit_cast(v8h, v4i{__builtin_bit_cast(v2i, v0).x, __builtin_bit_cast(v2i, v0).y,
                                         __builtin_bit_cast(v2i, v1).x, __builtin_bit_cast(v2i, v1).y});
    };
    auto p_op = [&](const _Float16* buf, int hb) -> v8h {
      return __builtin_bit_cast(v8h, *reinterpret_cast<const v4i*>(&buf[(hb * 16 + lq) * P_STRIDE + lg * 8]));
    };
    // the tile's p_lo flag (same in every lane; stable until the next tile)
    const bool lo = __builtin_amdgcn_readfirstlane(vflag_s[vb]) != 0u;
    if constexpr (HB <= 2) {
      // all V operands held; p_hi of each head block, then p_lo if needed
      v8h vv[NBLK];
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) vv[nb] = v_op(nb);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const v8h ph = p_op(pb, hb);
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb) {
          o[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, vv[nb], o[hb][nb], 0, 0, 0);
        }
      }
      if (lo) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const v8h pl = p_op(pbl, hb);
#pragma unroll
          for (int nb = 0; nb < NBLK; ++nb) o[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, vv[nb], o[hb][nb], 0, 0, 0);
        }
      }
    } else {
      // 64 heads: registers are short, so the p_lo pass reads V again
      v8h pv[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) pv[hb] = p_op(pb, hb);
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb) {
        const v8h vv = v_op(nb);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) o[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv[hb], vv, o[hb][nb], 0, 0, 0);
      }
      if (lo) {
        asm volatile("" ::: "memory");  // V is read again, not held in registers
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) pv[hb] = p_op(pbl, hb);
#pragma unroll
        for (int nb = 0; nb < NBLK; ++nb) {
          const v8h vv = v_op(nb);
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) o[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv[hb], vv, o[hb][nb], 0, 0, 0);
        }
      }
    }
  };

  // Tiles 0 and 1 are issued before the loop in the loop's own order, pinned
  // by scheduling barriers: the wait counter at the loop head merges this
  // entry with the back edge, so any other order would make each K step wait
  // for every load in flight.  The loop is unrolled by two (a register buffer
  // per parity); an odd last tile is followed by an all-masked one.
  LoadT buf0[KSTEPS], buf1[KSTEPS];
  int bm0, bm1;
  float4 sc0 = make_float4(0.f, 0.f, 0.f, 0.f), sc1 = sc0;  // FP8 row scales per parity
  {
    const LoadT* s0 = row_of(0, bm0);
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      buf0[c] = s0[c * 4];
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FP8) {
      sc0 = *scales_of(0);
      __builtin_amdgcn_sched_barrier(0);
    }
    const LoadT* s1 = row_of(1, bm1);
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      buf1[c] = s1[c * 4];
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FP8) {
      sc1 = *scales_of(1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (int t = 0; t < ntile; t += 2) {
    tile_step(t, buf0, bm0, sc0);
    tile_step(t + 1, buf1, bm1, sc1);
  }

  // ---- finish: per-head sums of the owned heads, then every wave's channels ----
  float l_tot = l_run + __shfl_xor(l_run, 8, 64);
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (own_tq == 0 && wave < NSW) {
    fin_s[0][own_h] = l_tot > 0.f ? m_ref : -INFINITY;
    fin_s[1][own_h] = l_tot;
  }
  // LDS-only barriers from here on: the loop leaves the (unused) loads of two
  // tiles past the end in flight, and a full barrier would wait for them
  lds_barrier();
  const int d_base = wave * OUT_DIM;
  if (P.splits == 1) {
    float* orow = P.out[layer] + ((size_t)r * ATT_HEADS + h0) * LAT_DIM;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float inv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float li = fin_s[1][hb * 16 + 4 * lg + i];
        inv[i] = li > 0.f ? 1.f / li : 0.f;
      }
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          orow[(size_t)(hb * 16 + 4 * lg + i) * LAT_DIM + d_base + nb * 16 + lq] = o[hb][nb][i] * inv[i];
    }
    if (P.lse[layer] && own_tq == 0 && wave < NSW)
      P.lse[layer][(size_t)r * ATT_HEADS + h0 + own_h] = l_tot > 0.f ? m_ref * LN2 + logf(l_tot) : -INFINITY;
  } else {
    // the split's normalised output O / l (a convex combination of latent
    // rows, so within their range), in fp16 when every value is below
    // PART_F16_MAX in magnitude -- staged in LDS (the V tiles are free now) and
    // written with 16-B stores -- otherwise in fp32 straight from registers
    const size_t part = unit;  // (layer, row, split)
    bool big = false;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float inv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float li = fin_s[1][hb * 16 + 4 * lg + i];
        inv[i] = li > 0.f ? 1.f / li : 0.f;
      }
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[hb][nb][i] *= inv[i];
          big |= !(fabsf(o[hb][nb][i]) < PART_F16_MAX);  // NaN counts as large
        }
    }
    // the fp16 copy is staged in any case; the barrier that publishes it also
    // publishes whether any value was too large for it
    if (__any(big) && lane == 0) big_s = 1u;
    _Float16* stage = &vt[0][0];
    static_assert(2 * TILE_TOK * V_STRIDE >= NH * LAT_DIM, "staging fits in the V tiles");
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          stage[(hb * 16 + 4 * lg + i) * LAT_DIM + d_base + nb * 16 + lq] = (_Float16)o[hb][nb][i];
    lds_barrier();
    const bool f32 = big_s != 0u;  // uniform
    char* slot = P.o_part + (part * ATT_HEADS + h0) * (LAT_DIM * 4);  // 2 KiB per head
    if (!f32) {
      constexpr int N16 = NH * LAT_DIM * 2 / 16;  // 16-B chunks, 64 per head
#pragma unroll
      for (int k = 0; k < N16 / MLA_THREADS; ++k) {
        const int c = tid + k * MLA_THREADS;
        *reinterpret_cast<v4i*>(slot + (size_t)(c >> 6) * (LAT_DIM * 4) + (c & 63) * 16) =
            reinterpret_cast<const v4i*>(stage)[c];
      }
    } else {
      float* base = reinterpret_cast<float*>(slot) + 4 * lg * LAT_DIM + d_base + lq;  // head 4lg, this lane's channel
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nb = 0; nb < NBLK; ++nb) base[(hb * 16 + i) * LAT_DIM + nb * 16] = o[hb][nb][i];
    }
    if (own_tq == 0 && wave < NSW) {
      float4* mp = reinterpret_cast<float4*>(P.ml_part) + (part * ATT_HEADS + h0 + own_h);
      *mp = make_float4(l_tot > 0.f ? m_ref : -INFINITY, l_tot, f32 ? 1.f : 0.f, 0.f);
    }
  }
}

// Merge the splits of one (row, head): split s weighs l_s 2^(m_s - M) / sum,
// applied to its normalised partial (128 threads x 4 channels, loads unrolled).
// NS > 0: exactly NS splits, and the partials' fp16 form (the common case) is
// loaded in the same round as the splits' statistics, saving one dependent
// round trip; if any partial turns out to be in fp32 it is read again below.
template <bool MULTI, int NS>
__global__ __launch_bounds__(128) void k_mla_combine(const MlaPtrs P, int32_t rows) {
  __shared__ float wsh[MAX_SPLITS];
  __shared__ uint32_t fsh[MAX_SPLITS];
  __shared__ float stat[3];
  const int rl = blockIdx.x / ATT_HEADS, h = blockIdx.x % ATT_HEADS;
  const int layer = MULTI ? rl / rows : 0;
  const int r = MULTI ? rl % rows : rl;
  const int S = P.splits;
  const size_t part0 = ((size_t)layer * rows + r) * S;  // (layer, row, split 0)
  const float4* ml = reinterpret_cast<const float4*>(P.ml_part) + (part0 * ATT_HEADS + h);
  const char* op = P.o_part + (part0 * ATT_HEADS + h) * (LAT_DIM * 4);
  constexpr size_t SPLIT_STRIDE = (size_t)ATT_HEADS * LAT_DIM * 4;
  v4h pre[NS > 0 ? NS : 1];
  if constexpr (NS > 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) pre[s] = *reinterpret_cast<const v4h*>(op + s * SPLIT_STRIDE + threadIdx.x * 8);
  }
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const float4 v = lane < S ? ml[(size_t)lane * ATT_HEADS] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
    const float m = v.x, l = v.y;
    const bool f32 = v.z != 0.f;
    float M = m;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float w = (M == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - M);
    float ws = w * l;
    for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o, 64);
    if (lane < S) {
      wsh[lane] = ws > 0.f ? w * l / ws : 0.f;  // weight of the normalised partial
      fsh[lane] = f32 ? 1u : 0u;
    }
    const bool any32 = __any(lane < S && f32);
    if (lane == 0) {
      stat[0] = M;
      stat[1] = ws;
      stat[2] = any32 ? 1.f : 0.f;
    }
  }
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (NS > 0 && stat[2] == 0.f) {  // uniform: every partial in fp16, already loaded
#pragma unroll
    for (int s = 0; s < (NS > 0 ? NS : 1); ++s) {
      const float f = wsh[s];
      acc.x = fmaf(f, (float)pre[s][0], acc.x);
      acc.y = fmaf(f, (float)pre[s][1], acc.y);
      acc.z = fmaf(f, (float)pre[s][2], acc.z);
      acc.w = fmaf(f, (float)pre[s][3], acc.w);
    }
  } else if (stat[2] == 0.f) {  // uniform: every partial in fp16
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
      const float f = wsh[s];
      const v4h v = *reinterpret_cast<const v4h*>(op + s * SPLIT_STRIDE + threadIdx.x * 8);
      acc.x = fmaf(f, (float)v[0], acc.x);
      acc.y = fmaf(f, (float)v[1], acc.y);
      acc.z = fmaf(f, (float)v[2], acc.z);
      acc.w = fmaf(f, (float)v[3], acc.w);
    }
  } else {
    for (int s = 0; s < S; ++s) {
      const float f = wsh[s];
      float4 x;
      if (fsh[s]) {  // uniform
        x = *reinterpret_cast<const float4*>(op + s * SPLIT_STRIDE + threadIdx.x * 16);
      } else {
        const v4h v = *reinterpret_cast<const v4h*>(op + s * SPLIT_STRIDE + threadIdx.x * 8);
        x = make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
      }
      acc.x = fmaf(f, x.x, acc.x);
      acc.y = fmaf(f, x.y, acc.y);
      acc.z = fmaf(f, x.z, acc.z);
      acc.w = fmaf(f, x.w, acc.w);
    }
  }
  *reinterpret_cast<float4*>(P.out[layer] + ((size_t)r * ATT_HEADS + h) * LAT_DIM + threadIdx.x * 4) = acc;
  if (P.lse[layer] && threadIdx.x == 0)
    P.lse[layer][(size_t)r * ATT_HEADS + h] = stat[1] > 0.f ? stat[0] * LN2 + logf(stat[1]) : -INFINITY;
}

MlaPlan plan_mla(int32_t rows, int32_t k, int32_t layers) {
  // about 256 workgroups in flight over all layers, at least 32 groups (four
  // 32-token tiles) per split
  MlaPlan p;
  p.rows = rows;
  const long long units = (long long)rows * layers;
  int s = (int)((256 + units - 1) / units);
  int smax = (k + 31) / 32;
  if (s > smax) s = smax;
  if (s > MAX_SPLITS) s = MAX_SPLITS;
  if (s < 1) s = 1;
  p.splits = s;
  p.groups_per_split = (k + s - 1) / s;
  return p;
}

isa_status launch_sparse_mla(const BatchArgs& a, const MlaPlan& p, int32_t n_layers, const uint16_t* const* q,
                             const void* const* latent, const float* const* lat_scale, const int32_t* bt,
                             const int32_t* row_seq,
                             const int32_t* row_pos, const int32_t* idx, const int32_t* count, int32_t k,
                             float sm_scale, float* const* out, float* const* lse, const MlaWs& w,
                             hipStream_t stream) {
  MlaPtrs P{};
  for (int l = 0; l < n_layers; ++l) {
    P.q[l] = q[l];
    P.latent[l] = latent[l];
    P.lat_scale[l] = lat_scale ? lat_scale[l] : nullptr;
    P.out[l] = out[l];
    P.lse[l] = lse ? lse[l] : nullptr;
  }
  P.n_layers = n_layers;
  P.rows = p.rows;
  P.bt = bt;
  P.row_seq = row_seq;
  P.row_pos = row_pos;
  P.idx = idx;
  P.count = count;
  P.o_part = w.o_part;
  P.ml_part = w.ml_part;
  P.err = w.err;
  P.k = k;
  P.c2 = sm_scale * LOG2E;
  P.splits = p.splits;
  P.gps = p.groups_per_split;
  const int units = n_layers * p.rows * p.splits;
  P.n_units = units;
  // a launch of at most 128 units would fill half the CUs: split the heads
  const bool hsplit = units <= 128;
  const int nx = device_info().n_xcd;
  P.n_xcd = nx;
  const dim3 grid(hsplit ? (unsigned)((units + nx - 1) / nx * nx * 2) : (unsigned)units), block(MLA_THREADS);
  hipError_t e;
#define ISA_MLA_LAUNCH(FP8_, MULTI_)                                                                         \
  (hsplit ? launch_timed(ISA_TIMER_MLA_SPLIT, k_mla_split<FP8_, MULTI_, ATT_HEADS / 2>, grid, block, stream, a, P) \
          : launch_timed(ISA_TIMER_MLA_SPLIT, k_mla_split<FP8_, MULTI_, ATT_HEADS>, grid, block, stream, a, P))
  if (lat_scale)  // the FP8 cache is attended one layer per call
    e = n_layers == 1 ? ISA_MLA_LAUNCH(true, false) : hipErrorInvalidValue;
  else
    e = n_layers > 1 ? ISA_MLA_LAUNCH(false, true) : ISA_MLA_LAUNCH(false, false);
#undef ISA_MLA_LAUNCH
  if (e != hipSuccess) return ISA_ERR_HIP;
  if (p.splits > 1) {
    const dim3 cgrid((unsigned)(n_layers * p.rows * ATT_HEADS)), cblock(128);
#define ISA_COMBINE(MULTI_)                                                                                  \
  switch (p.splits) {                                                                                        \
    case 2: hipLaunchKernelGGL((k_mla_combine<MULTI_, 2>), cgrid, cblock, 0, stream, P, p.rows); break;     \
    case 4: hipLaunchKernelGGL((k_mla_combine<MULTI_, 4>), cgrid, cblock, 0, stream, P, p.rows); break;     \
    case 8: hipLaunchKernelGGL((k_mla_combine<MULTI_, 8>), cgrid, cblock, 0, stream, P, p.rows); break;     \
    case 16: hipLaunchKernelGGL((k_mla_combine<MULTI_, 16>), cgrid, cblock, 0, stream, P, p.rows); break;   \
    default: hipLaunchKernelGGL((k_mla_combine<MULTI_, 0>), cgrid, cblock, 0, stream, P, p.rows); break;    \
  }
    if (n_layers > 1) {
      ISA_COMBINE(true)
    } else {
      ISA_COMBINE(false)
    }
#undef ISA_COMBINE
    if (hipGetLastError() != hipSuccess) return ISA_ERR_HIP;
  }
  return ISA_OK;
}

}  // namespace isa
