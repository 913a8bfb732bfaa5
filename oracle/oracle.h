/*
 * oracle.h -- plain, slow CPU oracle of the IndexPool sparse-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no source, header, table or
 * helper with the GPU library.
 *
 * Sources (web pages; cited by title and section):
 *  [WIKI]  "GLM-5.3-Flash: 하이브리드 희소·선형 어텐션과 IndexPool·EPD로 1M 컨텍스트를
 *          오픈 소스로 서빙하는 방법" (llm-wiki.hwlabs.dev) -- sections "IndexPool:
 *          인덱서 KV 캐시를 4배 압축" (the pooling equation), "희소 어텐션: 인덱서로
 *          필요한 토큰만", "양자화: W8A8와 혼합 캐시".
 *  [REMIO] "GLM-5.3 Sparse Attention은 연산량을 줄이지만 HBM 수요는 지속된다"
 *          (remio.ai) -- section "GLM-5.3 Sparse Attention이 실제로 바꾸는 것".
 *  [TREND] "GLM-5.3-Flash vs Qwen3.8-Flash-Next: 두 중국 AI 연구소가 독립적으로 같은
 *          모델 설계로 수렴한 이유" (alltoptrend.co.kr) -- sections "수렴점 2 — 4배
 *          압축 후 2,048 토큰만 유지" and "의견이 갈리는 지점 — 위치 인코딩".
 *
 * Fixed dimensions: indexer keys 128-d, 32 indexer heads, groups of 4 tokens,
 * 64 attention heads over a 512-d latent.  Integers are int64, floating point is
 * double.  Every function is reentrant (no global state), so callers may run
 * independent rows on separate threads.
 *
 * Parity unpinned (conventions no page fixes, shared by both sides): the
 * meaning of the learned pooling weights as one 4-vector per layer, the prefill
 * block-causal rule, and the input distributions.
 */
#ifndef ISA_ORACLE_H
#define ISA_ORACLE_H

#include <stdint.h>

#define OR_IDX_DIM 128
#define OR_IDX_HEADS 32
#define OR_GROUP 4
#define OR_ATT_HEADS 64
#define OR_LAT_DIM 512
#define OR_KDA_DIM 128

#ifdef __cplusplus
extern "C" {
#endif

/* IndexPool of one sequence ([WIKI] IndexPool section, pooling equation) then
 * symmetric int8 quantisation of the pooled cache ([WIKI] quantisation
 * section: the distant compressed cache is INT8).
 *   keys    bf16 bits, [L,128], logical token order
 *   w4      the 4 learned pooling weights (fp32, widened to double)
 *   pooled  [G,128] double pooled values before quantisation (may be NULL)
 *   k8      [G,128] int8 output, G = ceil(L/4)
 *   scale   fp32 output: amax/127 (1 when amax == 0)
 *   amax    double output (may be NULL)
 * Returns 0, or -1 for L < 1. */
int oracle_pool(const uint16_t* keys, int64_t L, const float* w4, double* pooled, int8_t* k8,
                float* scale, double* amax);

/* Same pooling, quantised with a scale given by the caller (clamped to +-127). */
int oracle_pool_given_scale(const uint16_t* keys, int64_t L, const float* w4, float scale, int8_t* k8);

/* Lightning-indexer scores of one query over G pooled groups ([REMIO] section on
 * what sparse attention changes: the indexer scores previous positions;
 * [TREND] convergence 2: 32 heads):
 *   S[g] = sum_h w[h] * max(0, sum_d q[h][d] * k8[g][d])
 *   q [32,128] int8, w [32] int8, k8 [G,128] int8, S [G] int64. */
void oracle_scores(const int8_t* q, const int8_t* w, const int8_t* k8, int64_t G, int64_t* S);

/* Prefill scores of a query at absolute position pos: as above for g <= pos/4,
 * and -1 (masked) for later groups. */
void oracle_prefill_scores(const int8_t* q, const int8_t* w, int64_t pos, const int8_t* k8, int64_t G,
                           int64_t* S);

/* Top-k selection ([REMIO]: top-k positions, dense below the budget; [TREND]
 * convergence 2: 512 blocks of 4 = 2048 tokens).  Valid groups are those with
 * S >= 0.  If at most K are valid all are selected; otherwise the first K under
 * the order (higher score first, then lower group index).  idx [K] is written
 * in ascending group order, padded with -1; *count = number selected. */
int oracle_topk(const int64_t* S, int64_t G, int32_t K, int32_t* idx, int32_t* count);

/* Softmax attention of one query row over the tokens of the selected groups
 * ([WIKI] sparse attention section: softmax only over the indexer's picks;
 * [REMIO]: MLA attends over compressed latent rows; [TREND] positional
 * encoding section: NoPE, no rotary part).  Absorbed MLA: keys = values = the
 * 512-d latent row.
 *   q    bf16 bits [64,512]; lat bf16 bits [L,512] (logical rows of the sequence)
 *   sel  [count] selected group ids; token t is used iff t/4 in sel, t < L and t <= pos
 *   out  [64,512] double; lse [64] double (natural log of the softmax denominator
 *        plus the max, -inf when no token is visible, out = 0 then). */
int oracle_attention(const uint16_t* q, const uint16_t* lat, int64_t L, int64_t pos, const int32_t* sel,
                     int32_t count, double scale, double* out, double* lse);

/* FP8 latent cache ([WIKI] quantisation section: the recent, high-importance
 * cache is kept in FP8).  The pages name no FP8 format or scaling; this oracle
 * follows the library's contract: OCP E4M3 (bias 7, subnormals, S.1111.111 =
 * NaN, no infinities, largest value 448) with one fp32 scale per latent row.
 *   decode: the value of a code (NaN for the two NaN codes)
 *   encode: nearest value, ties to the even mantissa; a value that rounds past
 *           448 (|x| > 464) becomes NaN (no saturation); NaN -> 0x7F
 *   oracle_latent_fp8: per row, amax over its 512 bf16 values (as fp32),
 *           scale = amax / 448 in fp32 (1 when amax == 0), code = encode(x / scale)
 *           with the division in fp32.  Returns -1 for a non-finite value.
 *   oracle_attention_fp8: oracle_attention with latent value scales[t] * decode(code). */
double oracle_fp8_decode(uint8_t c);
uint8_t oracle_fp8_encode(float x);
int oracle_latent_fp8(const uint16_t* lat, int64_t n, uint8_t* codes, float* scales);
int oracle_attention_fp8(const uint16_t* q, const uint8_t* codes, const float* scales, int64_t L, int64_t pos,
                         const int32_t* sel, int32_t count, double scale, double* out, double* lse);

/* One decode step of one head of a linear-attention (KDA) layer ([WIKI] linear
 * attention section: the delta update of the state matrix; [TREND] section on
 * the linear layers: KDA's channel-wise decay).  Reading: with S [128][128]
 * (row i = key channel, column j = value channel),
 *   S' = diag(alpha) S;  u = S'^T k;  S'' = S' + beta k (v - u)^T;  o = S''^T q;
 *   S := bf16(S'') rounded to nearest even.  With alpha = 1 this is the pages'
 *   S - beta k (k^T S) + beta k v^T.
 *   q, k, v  bf16 bits [128]; alpha fp32 [128]; beta fp32; S bf16 bits [128*128]
 *   (in/out); o double [128].  Returns -1 if the new state is not finite. */
int oracle_kda_step(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* alpha, float beta,
                    uint16_t* S, double* o);
/* Nearest bf16 of a double (ties to even), as bits. */
uint16_t oracle_bf16_round(double x);

#ifdef __cplusplus
}
#endif
#endif
