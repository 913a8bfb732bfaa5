/*
 * isa.h -- C ABI of the IndexPool sparse-attention path for AMD Instinct MI355X
 * (gfx950): IndexPool -> 32-head lightning indexer with top-512-group selection
 * -> NoPE MLA softmax attention over the selected latent rows.
 *
 * Sources (web pages; cited by title and section):
 *  [WIKI]  "GLM-5.3-Flash: 하이브리드 희소·선형 어텐션과 IndexPool·EPD로 1M 컨텍스트를
 *          오픈 소스로 서빙하는 방법" (llm-wiki.hwlabs.dev): sections "희소 어텐션:
 *          인덱서로 필요한 토큰만" (an indexer keeps one key per position and picks
 *          the positions softmax attention runs over), "IndexPool: 인덱서 KV 캐시를
 *          4배 압축" (pooling equation k_pool = sum_i w_i k_i over 4 consecutive
 *          keys, weights summing to 1, learned; a quarter of the storage), "양자화:
 *          W8A8와 혼합 캐시" (the distant compressed cache is INT8).
 *  [REMIO] "GLM-5.3 Sparse Attention은 연산량을 줄이지만 HBM 수요는 지속된다"
 *          (remio.ai), section "GLM-5.3 Sparse Attention이 실제로 바꾸는 것": the
 *          indexer scores earlier positions and keeps the top-k (2048); MLA
 *          attends over compressed latent rows; below 2048 positions attention
 *          stays dense; the indexer still has to see the whole history.
 *  [TREND] "GLM-5.3-Flash vs Qwen3.8-Flash-Next: 두 중국 AI 연구소가 독립적으로 같은
 *          모델 설계로 수렴한 이유" (alltoptrend.co.kr): section "수렴점 2 — 4배 압축
 *          후 2,048 토큰만 유지" (32-head lightning indexer, pooling before scoring,
 *          4-token blocks x top 512 = 2048 tokens) and section "의견이 갈리는 지점 —
 *          위치 인코딩" (qk_rope_head_dim = 0: NoPE).
 * The pages give no score formula, dtypes, tie rule or interface; the choices
 * made here are stated at each declaration.
 *
 * Conventions for every call
 *  - Fixed dimensions: indexer keys 128-d, 32 indexer heads, groups of 4 tokens,
 *    64 attention heads over a 512-d latent, k <= 512 groups.
 *  - Memory is owned by the caller.  Pointers marked [dev] are device pointers,
 *    [host] are host pointers read during the call only.  All [dev] pointers
 *    must be 16-byte aligned.  Tensors are dense row-major.
 *  - Paging: a page holds 256 tokens of indexer keys ([256,128] bf16, 64 KiB) or
 *    of latent rows ([256,512] bf16, 256 KiB), which is 64 pooled groups
 *    ([64,128] int8, 8 KiB).  Logical page j of a sequence is tokens
 *    256j..256j+255 = groups 64j..64j+63; one block table maps it to the same
 *    physical page id in the key, latent and pooled pools.
 *  - Work is enqueued on `stream`; no call synchronises or reads device memory
 *    on the host.  Outputs are valid once the stream reaches the call.
 *  - Workspace: `ws` [dev] of at least isa_workspace_size(...) bytes, zero-
 *    filled once before its first use (isa_workspace_init or any zero fill).
 *    Layout, the same for every call: the error word in the first 256 bytes,
 *    then the call's own scratch, which the call writes before it reads it:
 *    nothing but the error word carries over from one call to the next.  So
 *    one workspace may serve calls of any batch shape and be shared by
 *    different calls, provided it is as large as each call asks; calls that
 *    share a workspace must be ordered on one stream.
 *  - Errors: argument errors are reported synchronously by the return code
 *    before anything is enqueued.  Errors that depend on device data (a page
 *    id outside the pool, a head weight outside [0,64], a score above
 *    INT32_MAX, a row position outside its sequence) set bits in the sticky
 *    error word at the start of the workspace; read it with isa_device_error.
 *    Nothing aborts or throws across this boundary.
 */
#ifndef ISA_H
#define ISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* isa_stream_t; /* a hipStream_t (0 = the null stream) */

typedef enum {
  ISA_OK = 0,
  ISA_ERR_INVALID_ARG = 1,  /* NULL / misaligned pointer, bad size, bad flag */
  ISA_ERR_UNSUPPORTED = 2,  /* a size beyond what the library supports */
  ISA_ERR_WORKSPACE = 3,    /* workspace smaller than isa_workspace_size() */
  ISA_ERR_HIP = 4           /* the HIP runtime rejected a launch */
} isa_status;

/* bits of the device error word */
#define ISA_DERR_PAGE_OOB 0x1u       /* block-table entry outside [0, num_pages) */
#define ISA_DERR_HEADW_RANGE 0x2u    /* indexer head weight outside [0, 64] */
#define ISA_DERR_SCORE_OVERFLOW 0x4u /* an indexer score above INT32_MAX */
#define ISA_DERR_ROW_RANGE 0x8u      /* a row's sequence, position or selection count, a selected group
                                        id, or a prefill query position outside its sequence */
#define ISA_DERR_NONFINITE 0x10u     /* non-finite pooled amax (NaN / Inf indexer keys) */

#define ISA_MAX_BATCH 256          /* sequences per call */
#define ISA_MAX_SEQ_LEN (1 << 22)  /* tokens per sequence */
#define ISA_MAX_LAYERS 8           /* layers sharing one selection (isa_sparse_mla_decode_shared) */
#define ISA_MAX_K 512              /* groups selected per row */

/* One batch of sequences that share page pools. */
typedef struct {
  int32_t batch;                /* B, 1..ISA_MAX_BATCH */
  int32_t max_pages;            /* columns of block_table; >= ceil(L_b/256) for every b */
  int32_t num_pages;            /* physical pages in each pool (bounds for block_table) */
  int32_t reserved;             /* must be 0 */
  const int32_t* seq_lens_host; /* [host] [B] tokens per sequence, 1..ISA_MAX_SEQ_LEN */
  const int32_t* block_table;   /* [dev]  [B, max_pages] physical page ids */
} isa_seqs;

enum {
  ISA_OP_INDEXPOOL = 1,
  ISA_OP_INDEXER_TOPK = 2,
  ISA_OP_SPARSE_MLA = 3,
  ISA_OP_PREFILL_SCORES = 4,
  ISA_OP_APPEND_TOKEN = 5,
  ISA_OP_LATENT_FP8 = 6,
  ISA_OP_KDA_STEP = 7
};

/* Workspace bytes (a multiple of 256) that `op` needs for these sequences.
 * rows: query rows (attention and top-k from precomputed scores; ignored
 * otherwise); cols: for ISA_OP_SPARSE_MLA the number of layers attended in one
 * call of isa_sparse_mla_decode_shared (0 or 1 for isa_sparse_mla_decode),
 * ignored otherwise.  Returns 0 for invalid arguments. */
size_t isa_workspace_size(int op, const isa_seqs* s, int32_t rows, int32_t cols);

/* Zero-fill a workspace on `stream` (needed once, before its first use). */
isa_status isa_workspace_init(void* ws, size_t ws_bytes, isa_stream_t stream);

/* Copy the sticky device error word to *err_word [host] (synchronises
 * `stream`), and clear it when `clear` is nonzero. */
isa_status isa_device_error(void* ws, isa_stream_t stream, uint32_t* err_word, int clear);

const char* isa_status_string(isa_status status);
const char* isa_version(void);

/* Kernel timing hook, for benchmarks.  `starts` and `stops` [host] are arrays
 * of n hipEvent_t handles, or NULL with n = 0 to switch the hook off.  While it
 * is set, the i-th later launch of `kernel` (counting from this call) is
 * dispatched with starts[i % n] / stops[i % n] as its start and stop events
 * (hipExtLaunchKernelGGL), so hipEventElapsedTime gives that kernel's own
 * execution time.  The
 * arrays are copied (at most 4096 pairs); the events stay the caller's.  The
 * setting is process-wide and not thread-safe.  ISA_ERR_INVALID_ARG for an
 * unknown kernel id, n outside 0..4096 or a NULL handle. */
#define ISA_TIMER_INDEXER_SCORE 1 /* scoring kernel of isa_indexer_topk (decode mode) */
#define ISA_TIMER_MLA_SPLIT 2     /* main kernel of isa_sparse_mla_decode */
isa_status isa_set_kernel_timer(int32_t kernel, void* const* starts, void* const* stops, int32_t n);

/* Read-bandwidth probe, for benchmarks: reads every byte of `buf` ([dev],
 * `bytes` a nonzero multiple of 16) once, one workgroup per CU streaming a
 * contiguous share in 4-KiB chunks of wave-wide non-temporal 16-byte loads
 * (the decode scoring stream's access shape).  *sink ([dev] uint32) is written only if the XOR of all words
 * read equals 0x9E3779B9 (so that no load is dropped).  Its rate over a buffer
 * larger than the on-package caches is the practical HBM read ceiling the
 * kernels' rates can be set against.  clocks ([dev] uint64 [2], or NULL)
 * receives the shader clock cycles (s_memtime) and 100 MHz reference ticks
 * (s_memrealtime) that one wave spent, whose ratio is the shader clock. */
isa_status isa_read_probe(const void* buf, size_t bytes, uint32_t* sink, uint64_t* clocks, isa_stream_t stream);

#define ISA_SCALE_DYNAMIC 0u /* scales[b] := max|pooled| / 127 of sequence b (1 if all zero) */
#define ISA_SCALE_GIVEN 1u   /* use scales[b] as given (> 0), single pass, clamp to +-127 */

/*
 * (1) IndexPool + int8 quantisation of the indexer key cache ([WIKI] IndexPool
 * and quantisation sections; [TREND] convergence 2: pooling precedes scoring).
 *   keys    [dev] bf16 bits [num_pages, 256, 128], token-paged
 *   w4      [host] the 4 learned pooling weights (fp32, sum 1), shared by all
 *           groups and channels
 *   s       sequences and block table
 *   scales  [dev] fp32 [B]: written (DYNAMIC) or read (GIVEN)
 *   pooled  [dev] int8 [num_pages, 64, 128], group-paged; group g of sequence b is
 *           row g%64 of page block_table[b][g/64]
 * Group g pools tokens 4g..4g+3: sum_i w_i k_{4g+i} in fp32.  A last group of
 * r < 4 tokens uses w_0..w_{r-1} divided by their sum.  The pooled value x is
 * stored as clamp(round_half_even(x / scale), -127, 127).  Rows of a sequence's
 * last page beyond its last group are left untouched.
 */
isa_status isa_indexpool(const uint16_t* keys, const float* w4, const isa_seqs* s, float* scales,
                         int8_t* pooled, uint32_t flags, void* ws, size_t ws_bytes, isa_stream_t stream);

/*
 * (2) Lightning-indexer scoring and top-k group selection ([REMIO] section on
 * what sparse attention changes: score earlier positions, keep the top-k,
 * dense below the budget; [TREND] convergence 2: 32 heads, 512 groups of 4).
 *
 * Decode mode (scores_in == NULL): one row per sequence, rows == s->batch.
 *   q       [dev] int8 [B, 32, 128] indexer query of each sequence
 *   head_w  [dev] int8 [B, 32] head weights, each in [0, 64]
 *   pooled  [dev] int8 [num_pages, 64, 128] (from isa_indexpool)
 *   score of group g:  S = sum_h head_w[h] * max(0, sum_d q[h][d] * pooled[g][d]),
 *   exact integer arithmetic; every group 0..ceil(L_b/4)-1 is a candidate.
 *   scores_out [dev] optional int32 [B, ld_scores] (ld_scores >= max_b ceil(L_b/4)):
 *           the scores of every group, for checking; NULL to skip.
 * Precomputed mode (scores_in != NULL, e.g. from isa_indexer_prefill_scores):
 *   scores_in [dev] int32 [rows, ld_scores]; entry < 0 means "not a candidate";
 *   q, head_w, pooled, scores_out are ignored and s may be NULL.
 *
 * Selection (both modes): the candidates of a row are ranked by higher score,
 * then lower group id; the first k are selected, or all candidates when there
 * are at most k (the dense fallback: fewer than 4k = 2048 tokens).
 *   out_idx   [dev] int32 [rows, k]: selected group ids in ascending order, then -1
 *   out_count [dev] int32 [rows]: number selected
 * k: 1..512 (512 = 2048 tokens).
 * Device errors (decode mode): ISA_DERR_HEADW_RANGE for a head weight outside
 * [0, 64]; ISA_DERR_SCORE_OVERFLOW for a score above INT32_MAX (scores are
 * accumulated in 32-bit unsigned arithmetic, which holds the largest possible
 * score -- 32 * 64 * 128 * 128 * 127 = 4,261,412,864 for any int8 query and
 * pooled entries within +-127, the range isa_indexpool and isa_append write
 * -- so the selection still ranks it exactly; scores_out holds it wrapped to
 * a negative int32); ISA_DERR_PAGE_OOB.  Pooled entries of -128 (never written
 * by this library) can, with a query of -128 on every channel, reach 2^32,
 * which wraps to 0 unreported.
 */
isa_status isa_indexer_topk(const int8_t* q, const int8_t* head_w, const int8_t* pooled, const isa_seqs* s,
                            const int32_t* scores_in, int32_t rows, int32_t ld_scores, int32_t k,
                            int32_t* out_idx, int32_t* out_count, int32_t* scores_out, void* ws,
                            size_t ws_bytes, isa_stream_t stream);

/*
 * (2b) isa_indexer_topk in decode mode for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The scratch the call needs lives in a device array inside
 * the library, ISA_NOALLOC_TOPK_BYTES bytes on each GPU the library runs on,
 * held until the process ends; nothing is allocated or freed by the call.
 * Arguments and results as isa_indexer_topk decode mode (rows = s->batch),
 * except:
 *   err_word [dev] one uint32 that receives the call's device error bits
 *            (ISA_DERR_*, OR-ed in: zero it before the first call)
 * ISA_ERR_UNSUPPORTED when the batch needs more scratch than the array holds,
 * i.e. when isa_workspace_size(ISA_OP_INDEXER_TOPK, s, 0, 0) exceeds
 * ISA_NOALLOC_TOPK_BYTES (at most 384 scoring work tiles: 8 sequences of 2^20
 * tokens, 64 of 2^17 and the ragged 32-sequence batch fit).  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results; order them on one
 * stream.  Nothing in the array has to start at zero: a call writes every
 * part of it that it reads.
 */
#define ISA_NOALLOC_TOPK_BYTES (256u + 384u * (8u + 8192u + 68096u))
isa_status isa_indexer_topk_noalloc(const int8_t* q, const int8_t* head_w, const int8_t* pooled, const isa_seqs* s,
                                    int32_t k, int32_t* out_idx, int32_t* out_count, int32_t* scores_out,
                                    int32_t ld_scores, uint32_t* err_word, isa_stream_t stream);

/*
 * (3) Sparse MLA attention over the selected groups ([WIKI] sparse attention
 * section: softmax only over the selected positions; [REMIO]: MLA keeps one
 * compressed latent per token; [TREND] positional encoding section: NoPE).
 * Absorbed form: keys = values = the 512-d latent row; no rotary part.
 *   q        [dev] bf16 bits [rows, 64, 512]
 *   latent   [dev] bf16 bits [num_pages, 256, 512], token-paged; values must be
 *            finite with magnitude below 65504 (they are converted to fp16)
 *   row_seq  [dev] int32 [rows] sequence of each row, or NULL: row r is sequence r
 *   row_pos  [dev] int32 [rows] last visible token, or NULL: L_seq - 1
 *   idx, count [dev] from isa_indexer_topk ([rows, k], [rows])
 *   sm_scale softmax scale (1/sqrt(512) for this model)
 *   out      [dev] fp32 [rows, 64, 512]: softmax(q_h . c_t * sm_scale) weighted sum of
 *            c_t over tokens t of the selected groups with t <= pos and t < L
 *   lse      [dev] fp32 [rows, 64] natural log-sum-exp of the scaled scores, or NULL
 * A row with no visible token gets out = 0 and lse = -inf.
 * Arithmetic: bf16 products with fp32 accumulation for q.c; fp32 softmax;
 * latents converted exactly to fp16 for the weighted sum, each probability
 * carried as two fp16 terms (p_hi = fp16(p), p_lo = fp16(p - p_hi), about
 * 2^-22 relative together), fp32 accumulation.  When a row's selection is
 * split over several workgroups, each split's normalised output (a convex
 * combination of latent rows) is held in fp16 when all of the workgroup's
 * values are below 16 in magnitude, else in fp32, and the splits are merged
 * with fp32 weights.  Accuracy against exact arithmetic: for latent values up
 * to 1024 in magnitude every output element is within 2e-2 (the rounding of
 * fp32 accumulation grows with the largest value beyond that) and lse within
 * 1e-3.  Device errors: ISA_DERR_ROW_RANGE for a bad row sequence, position,
 * count or group id (the row attends only to valid groups; none: out = 0),
 * ISA_DERR_PAGE_OOB.
 */
isa_status isa_sparse_mla_decode(const uint16_t* q, const uint16_t* latent, const isa_seqs* s,
                                 const int32_t* row_seq, const int32_t* row_pos, int32_t rows,
                                 const int32_t* idx, const int32_t* count, int32_t k, float sm_scale,
                                 float* out, float* lse, void* ws, size_t ws_bytes, isa_stream_t stream);

/*
 * (5) IndexShare: the attention of n_layers layers that reuse one selection
 * ([REMIO] section on IndexShare: one indexer per group of four sparse
 * attention layers; the other layers of the group attend over the positions it
 * selected).  One call does what n_layers calls of isa_sparse_mla_decode with
 * the same idx, count, rows, positions and block table would do, each layer
 * with its own query and latent pool (same page geometry, same block table);
 * the selected rows' page translation is done once for all layers.
 *   n_layers      1..ISA_MAX_LAYERS
 *   q, latent, out  [host] arrays of n_layers device pointers, each laid out as
 *                 the single-layer call's argument of the same name
 *   lse           NULL, or [host] array of n_layers device pointers (none NULL)
 * Other arguments, results and errors as isa_sparse_mla_decode; the workspace
 * is isa_workspace_size(ISA_OP_SPARSE_MLA, s, rows, n_layers).
 */
isa_status isa_sparse_mla_decode_shared(int32_t n_layers, const uint16_t* const* q, const uint16_t* const* latent,
                                        const isa_seqs* s, const int32_t* row_seq, const int32_t* row_pos,
                                        int32_t rows, const int32_t* idx, const int32_t* count, int32_t k,
                                        float sm_scale, float* const* out, float* const* lse, void* ws,
                                        size_t ws_bytes, isa_stream_t stream);

/*
 * (4) Prefill indexer scores of Q queries of one sequence (s->batch == 1)
 * against all its pooled groups -- a dense int8 contraction ([REMIO]: the
 * indexer scores the whole retained history).
 *   q       [dev] int8 [Q, 32, 128]; head_w [dev] int8 [Q, 32] in [0, 64]
 *   q_pos   [dev] int32 [Q] absolute token position of each query, in [0, L)
 *   scores  [dev] int32 [Q, ld_scores], ld_scores >= ceil(L/4): the decode score
 *           formula for groups g <= q_pos/4 (the query's own group included) and
 *           -1 for later groups and for columns ceil(L/4) .. ld_scores-1, so a
 *           whole row can go to isa_indexer_topk's precomputed mode.
 * Device errors: ISA_DERR_HEADW_RANGE for a head weight outside [0, 64];
 * ISA_DERR_ROW_RANGE for a position outside [0, L) (that query's row is all
 * -1); ISA_DERR_SCORE_OVERFLOW for a score above INT32_MAX (stored as a
 * negative number, so the row top-k would skip it); ISA_DERR_PAGE_OOB.
 */
isa_status isa_indexer_prefill_scores(const int8_t* q, const int8_t* head_w, const int32_t* q_pos, int32_t Q,
                                      const int8_t* pooled, const isa_seqs* s, int32_t* scores,
                                      int32_t ld_scores, void* ws, size_t ws_bytes, isa_stream_t stream);

/*
 * (6) Decode-time cache maintenance: append one token to every sequence of the
 * batch ([WIKI] IndexPool section: the indexer keeps one key per position and
 * four consecutive keys pool into one; this call keeps the pooled cache in step
 * as tokens arrive).  s->seq_lens_host holds the lengths AFTER the append
 * (L_b >= 1): the new token sits at position L_b - 1, on logical page
 * (L_b - 1) / 256, which the block table must map (the caller owns page
 * allocation; a token at a multiple of 256 starts a new page).
 *   key_new    [dev] bf16 bits [B, 128]: the new tokens' indexer keys
 *   latent_new [dev] bf16 bits [B, 512], or NULL to leave the latent pool alone
 *   w4         [host] fp32[4] pooling weights (as isa_indexpool)
 *   scales     [dev] fp32 [B]: each sequence's fixed quantisation scale, e.g.
 *              from an earlier isa_indexpool; used, never changed
 *   keys       [dev] bf16 bits [num_pages, 256, 128]: the key is written at the new token
 *   latent     [dev] bf16 bits [num_pages, 256, 512] (NULL iff latent_new is NULL)
 *   pooled     [dev] int8 [num_pages, 64, 128]: group (L_b - 1) / 4 is pooled
 *              again from its r = (L_b - 1) % 4 + 1 tokens (r < 4: the tail rule
 *              of isa_indexpool) and quantised with scales[b], clamped to +-127
 * After any sequence of appends the pooled cache equals what isa_indexpool with
 * ISA_SCALE_GIVEN and the same scales writes for the extended sequences (same
 * arithmetic, bit for bit).  Workspace: isa_workspace_size(ISA_OP_APPEND_TOKEN,
 * ...) bytes (the error word).  Device errors: ISA_DERR_PAGE_OOB for an unmapped
 * page (nothing written for that sequence), ISA_DERR_NONFINITE for a scale that
 * is not positive and finite (1 is used).
 */
isa_status isa_append_token(const uint16_t* key_new, const uint16_t* latent_new, const float* w4, const isa_seqs* s,
                            const float* scales, uint16_t* keys, uint16_t* latent, int8_t* pooled, void* ws,
                            size_t ws_bytes, isa_stream_t stream);

/*
 * (7) FP8 latent cache ([WIKI] quantisation section: the recent, high-importance
 * cache is kept in FP8).  The pages name no format; this library's contract:
 * OCP E4M3 codes (bias 7, subnormals, S.1111.111 = NaN, largest value 448) with
 * one fp32 scale per latent row.
 *
 * isa_latent_to_fp8 quantises every row t < L_b of the batch's sequences:
 * scale = amax / 448 over the row's 512 bf16 values (1 for a zero row), code =
 * nearest E4M3 value of x / scale (ties to even; the division in fp32).
 *   latent     [dev] bf16 bits [num_pages, 256, 512]
 *   codes      [dev] uint8 [num_pages, 256, 512] (rows of the sequences written)
 *   row_scales [dev] fp32 [num_pages, 256]
 * Workspace: isa_workspace_size(ISA_OP_LATENT_FP8, ...) bytes.  A non-finite
 * latent value sets ISA_DERR_NONFINITE.
 *
 * isa_sparse_mla_decode_fp8 is isa_sparse_mla_decode over such a cache: the
 * latent value of token t is row_scales[t] * decode(codes[t]).  Arithmetic:
 * codes decoded exactly to fp16, the query converted to fp16, fp16 products with
 * fp32 accumulation; the row scale multiplies the fp32 score and is folded into
 * the probability of the P.V product (carried as two fp16 terms, as above).  Row scales must be positive, finite
 * and at most 128.  Arguments, results and errors otherwise as
 * isa_sparse_mla_decode (same workspace size).
 */
isa_status isa_latent_to_fp8(const uint16_t* latent, const isa_seqs* s, uint8_t* codes, float* row_scales, void* ws,
                             size_t ws_bytes, isa_stream_t stream);
isa_status isa_sparse_mla_decode_fp8(const uint16_t* q, const uint8_t* codes, const float* row_scales,
                                     const isa_seqs* s, const int32_t* row_seq, const int32_t* row_pos, int32_t rows,
                                     const int32_t* idx, const int32_t* count, int32_t k, float sm_scale, float* out,
                                     float* lse, void* ws, size_t ws_bytes, isa_stream_t stream);

/*
 * (8) One decode step of a linear-attention (KDA) layer for n (sequence, head)
 * units ([WIKI] linear attention section: the state matrix's delta update
 * S_t = S_{t-1} - beta k (k^T S_{t-1}) + beta k v^T, and quantisation section:
 * the state stays BF16; [TREND] section on the linear layers: KDA's decay gate
 * is channel-wise).  Contract (the pages give no more): per unit, with the
 * state S [128][128] (row = key channel, column = value channel)
 *   S' = diag(alpha) S;  u = S'^T k;  S'' = S' + beta k (v - u)^T;  out = S''^T q
 * and S is replaced by S'' rounded to bf16 (nearest even).
 *   q, k, v [dev] bf16 bits [n, 128]; alpha [dev] fp32 [n, 128] decay per key
 *   channel; beta [dev] fp32 [n]; state [dev] bf16 bits [n, 128, 128], updated in
 *   place; out [dev] fp32 [n, 128].  No normalisation of k is applied.
 * Arithmetic in fp32.  Workspace: isa_workspace_size(ISA_OP_KDA_STEP, ...)
 * bytes.  A non-finite new state sets ISA_DERR_NONFINITE.
 */
isa_status isa_kda_decode_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha,
                               const float* beta, uint16_t* state, float* out, int32_t n, void* ws, size_t ws_bytes,
                               isa_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ISA_H */
