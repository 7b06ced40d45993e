/*
 * dsa.h -- C ABI of the DSA (lightning indexer + top-k + sparse MLA) hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * The method, as "TokenSpeed Kimi K3.1" (section "Integrating sparse attention
 * with the K3 stack") lays it out, runs per attention layer in four steps:
 * Write the new token's FP8 index key, Score every cached key with the
 * indexer's 32 heads, Select the 2,048 highest-scoring positions per query
 * row, and Attend with MLA over only those latent rows. This library covers
 * all four.
 *
 * Conventions shared by every entry point
 *  - Pointers are device pointers unless a comment says "host". `stream` is a
 *    hipStream_t passed as void* (NULL = the default stream). All work is
 *    enqueued asynchronously on that stream; nothing synchronises the host.
 *  - The caller owns every buffer, workspace included. The library never
 *    allocates or frees memory and keeps no pointer after a call returns.
 *    Between calls it holds only read-only facts about the device (scorer
 *    occupancy, compute-unit count), the message of the last error (per
 *    thread), and the device array of dsa_sparse_mla_decode_noalloc;
 *    calls on different streams with disjoint outputs and workspaces may
 *    run concurrently (dsa_sparse_mla_decode_noalloc calls on one device
 *    excepted).
 *  - Errors are returned as dsa_status codes, never thrown. Arguments are
 *    checked on the host before anything is enqueued; on any error nothing is
 *    enqueued. DSA_ERR_HIP reports a failed launch (see dsa_last_error()).
 *  - Rows are request-major: row = b * rows_per_request + r. Row r of request
 *    b sits at position ctx_len[b] - rows_per_request + r and sees the tokens
 *    0..position, its own token included (the Write step precedes Score).
 *    Decode verification rows and prefill chunks follow the same rule.
 *  - FP8 is the OCP E4M3 encoding (bias 7, max 448, no infinities).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent sizes */
  DSA_ERR_UNSUPPORTED = -2, /* a shape this build does not implement */
  DSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than dsa_workspace_size() */
  DSA_ERR_HIP = -4          /* a HIP launch failed; nothing else was enqueued after it */
} dsa_status;

enum { DSA_Q_BF16 = 0, DSA_Q_FP8 = 1 };

/* Index-key formats of a cache (dsa_cache.key_format). */
enum { DSA_KEY_FP8 = 0, DSA_KEY_MXFP4 = 1 };

/* Workspace kinds for dsa_workspace_size(). */
enum { DSA_WS_TOPK = 1, DSA_WS_MLA_DECODE = 2, DSA_WS_MLA_PREFILL = 3, DSA_WS_DECODE = 4 };
/* Workspace kinds for dsa_dcp_workspace_size(). */
enum { DSA_WS_DCP_TOPK = 5, DSA_WS_DCP_MLA = 6 };

#define DSA_BLOCK 64        /* tokens per cache page */
#define DSA_IDX_HEADS 32    /* indexer heads */
#define DSA_IDX_DIM 128     /* indexer head dim */
#define DSA_LAT_DIM 576     /* latent width: 512 compressed KV + 64 RoPE dims */
#define DSA_V_DIM 512       /* value width: the first 512 latent dims */
#define DSA_MLA_HEADS 16    /* MLA heads per call */
#define DSA_MAX_TOPK 2048

/*
 * Paged cache, split planes, 64-token pages. One page id addresses the same
 * 64 tokens in all four planes ("TokenSpeed Kimi K3.1", section "Storing index
 * keys in the flat KV cache": the index-key plane sits next to the latent
 * rows and shares their page).
 *   key_fp8   [num_blocks][64][128] E4M3 index keys (128 B per token)
 *   key_scale [num_blocks][64]      fp32 per-token key scale (4 B)
 *   lat_fp8   [num_blocks][64][576] E4M3 latent rows
 *   lat_scale [num_blocks][64]      fp32 per-token latent scale
 * A key or latent dequantises as code value * scale. Planes must be 16-byte
 * aligned.
 *
 * With key_format DSA_KEY_MXFP4 the index keys are MXFP4 instead, 68 B per
 * token ("vLLM Day-0 Support for Kimi K3.1 Pro", section "Native MXFP4
 * indexer": 68 bytes including scales in place of 132; "Inside vLLM's
 * hybrid KV cache" lists both widths), and key_fp8 / key_scale are unused:
 *   key_fp4   [num_blocks][64][64] E2M1 codes, two per byte: dim 2i in the
 *             low nibble of byte i, dim 2i + 1 in the high nibble
 *   key_e8m0  [num_blocks][64][4]  E8M0 scale of dims 32j .. 32j + 31
 * A key dim dequantises as E2M1(code) * 2^(scale - 127) (OCP MX: blocks of
 * 32 values sharing one power-of-two scale). Scale byte 255 (NaN) is not
 * supported.
 */
typedef struct {
  const uint8_t* key_fp8;
  const float* key_scale;
  const uint8_t* lat_fp8;
  const float* lat_scale;
  int32_t num_blocks;
  int32_t block_size; /* must be 64 */
  int32_t key_format; /* DSA_KEY_FP8 (0, the default) or DSA_KEY_MXFP4 */
  const uint8_t* key_fp4;
  const uint8_t* key_e8m0;
} dsa_cache;

/*
 * A batch of requests over the cache.
 *   ctx_len     device int32 [num_requests]: context length of each request,
 *               counting its rows_per_request new rows; rows_per_request <=
 *               ctx_len[b] <= max_ctx.
 *   block_table device int32 [num_requests][max_blocks]: page id of each
 *               64-token logical block; entries past a request's length may
 *               hold anything (-1 by convention) and are never read.
 *   max_blocks  host: row stride of block_table; max_blocks*64 >= max_ctx.
 *   max_ctx     host: an upper bound of every ctx_len (sizes the launch grid).
 */
typedef struct {
  int32_t num_requests;
  int32_t rows_per_request;
  const int32_t* ctx_len;
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t max_ctx;
} dsa_batch;

/*
 * Write: the new tokens' index keys into the cache ("TokenSpeed Kimi K3.1",
 * section "Integrating sparse attention with the K3 stack", step 1: the new
 * token's index key is normalised, quantised to FP8 with a single scale and
 * written into the cache; LayerNorm is the only key normalisation the loader
 * accepts). For row = b * rows_per_request + r, at position
 * p = ctx_len[b] - rows_per_request + r:
 *   y = LayerNorm(k[row]) over its 128 dims (biased variance, eps added to
 *       the variance) * ln_weight + ln_bias, computed in fp32;
 *   scale = max |y| / 448 (1 for an all-zero row);
 *   key_fp8[slot][0..127] = E4M3(y / scale) (round to nearest even),
 *   key_scale[slot] = scale, with slot = block_table[b][p / 64] * 64 + p % 64.
 *   k          bf16 [rows][128] (4-byte aligned)
 *   ln_weight, ln_bias  fp32 [128] (8-byte aligned)
 *   key_fp8    [num_blocks][64][128] E4M3, written; key_scale [num_blocks][64]
 * A row whose position is negative or whose page id lies outside
 * [0, num_blocks) is skipped (nothing is written for it). Only the new rows'
 * slots are written. eps must be positive and finite.
 */
int32_t dsa_index_key_write(const dsa_batch* batch, const void* k, const float* ln_weight, const float* ln_bias,
                            float eps, uint8_t* key_fp8, float* key_scale, int32_t num_blocks, void* stream);

/*
 * Score: the lightning indexer. For every row and every token s the row sees,
 *   scores[row * ld + s] = sum_h w[row][h] * ReLU(q[row][h] . khat_s)
 * with khat_s the dequantised key of token s (FP8: key_fp8[s] * key_scale[s];
 * MXFP4: each dim's E2M1 value times its block's power of two) and q[row][h] the row's query for
 * head h (DeepSeek-V3.2 form, to which "vLLM Day-0 Support for Kimi K3.1
 * Pro", section "What Kimi K3.1 Pro changes", points; 32 heads x 128 dims,
 * 132-byte FP8 keys). Each key is read once for all rows of its request
 * ("TokenSpeed Kimi K3.1", section "Reducing indexer overhead on AMD
 * MI350X").
 *   q        q_dtype DSA_Q_BF16: bf16 [rows][32][128];
 *            q_dtype DSA_Q_FP8:  E4M3 [rows][32][128] with q_scale fp32 [rows]
 *            (each row dequantises as code * q_scale[row]); q_scale must be
 *            NULL for BF16.
 *   w        bf16 [rows][32] head weights (any sign).
 *   scores   fp32 [rows][ld], ld >= max_ctx. Entries s > position(row) are not
 *            written.
 * key_scale and q_scale must be positive and finite: they live in device
 * memory, so the host cannot check them, and the kernels apply them after
 * the ReLU (ReLU(c x) = c ReLU(x) holds for c > 0 only).
 * Accumulation is fp32. E4M3 query values times E4M3 or E2M1 key values are
 * exact products. A bf16 query head enters as two E4M3 terms under one
 * power-of-two scale that puts the head's largest magnitude m in
 * (224, 448]; their sum reproduces every element whose magnitude is at
 * least about m * 2^-10 exactly, and smaller elements to within
 * m * 2^-10 / 224 (about 4.4e-6 m), so a head's dot product is off by at
 * most 4.4e-6 * m * sum_d |khat_s[d]|.
 */
int32_t dsa_index_score(const dsa_batch* batch, const dsa_cache* cache, const void* q, int32_t q_dtype,
                        const float* q_scale, const void* w, float* scores, int64_t ld, void* stream);

/*
 * Select: per row, the k highest scores among scores[row * ld + 0 .. row_len[row]-1]
 * ("TokenSpeed Kimi K3.1", step 3: a radix top-k keeps the 2,048
 * highest-scoring positions for each query). The selection is exact: ranking
 * is by fp32 score, -0 ranks equal to +0, and equal scores go to the lower
 * position, so the selected set is unique and identical across runs.
 *   row_len  device int32 [rows], 0 <= row_len[row] <= ld.
 *   idx      int32 [rows][k]: the selected positions in unspecified order;
 *            if row_len < k the first row_len entries hold every position and
 *            the rest are -1.
 *   ws       workspace of at least dsa_workspace_size(DSA_WS_TOPK, rows, ld, k, 0) bytes.
 * 1 <= k <= 2048. Scores must not be NaN.
 */
int32_t dsa_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t rows, int32_t k,
                 int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Attend: exact MLA over the selected latent rows only ("vLLM Day-0 Support
 * for Kimi K3.1 Pro", section "What Kimi K3.1 Pro changes": MLA runs exactly
 * over only the selected tokens; latent = 512 compressed KV + 64 RoPE dims,
 * "Kimi K3.1 Pro on AMD Instinct", model overview). For each row and head h:
 *   logit_j = softmax_scale * q[row][h] . chat_j  over all 576 dims,
 *   out[row][h][v] = sum_j softmax(logit)_j * chat_j[v]  for v < 512,
 *   lse[row][h] = log(sum_j exp(logit_j))  (natural log),
 * with chat_j = lat_fp8[j] * lat_scale[j] and j over idx[row][0..k-1];
 * entries < 0 are skipped. A row with no valid entry gets out = 0 and
 * lse = -inf. Positions index the row's request through block_table.
 *   q        bf16 [rows][num_heads][576]
 *   idx      int32 [rows][k], each entry -1 or a position the row sees.
 *   out      bf16 [rows][num_heads][512]
 *   lse      fp32 [rows][num_heads] or NULL.
 *   ws       workspace of dsa_workspace_size(DSA_WS_MLA_DECODE or _PREFILL, rows, 0, k, num_heads).
 * num_heads == 16, 1 <= k <= 2048. The decode variant splits each row's k
 * positions over several workgroups and merges them by log-sum-exp; the
 * prefill variant gives each row one workgroup.
 * The logits use the bf16 query as two E4M3 terms under one power-of-two
 * scale per head, as the indexer does (see dsa_index_score): elements more
 * than about 2^10 below the head's largest magnitude m carry an error of at
 * most about 4.4e-6 m. Probabilities and values multiply in bf16 with fp32
 * accumulation.
 */
int32_t dsa_sparse_mla_decode(const dsa_batch* batch, const dsa_cache* cache, const void* q, int32_t num_heads,
                              const int32_t* idx, int32_t k, float softmax_scale, void* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream);
int32_t dsa_sparse_mla_prefill(const dsa_batch* batch, const dsa_cache* cache, const void* q, int32_t num_heads,
                               const int32_t* idx, int32_t k, float softmax_scale, void* out, float* lse,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_sparse_mla_decode without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. Same arguments and results as
 * dsa_sparse_mla_decode, minus ws / ws_bytes. The split partials go to a
 * 16 MiB array of the library's own device memory (a static device array:
 * every GPU the library runs on holds one copy until the process ends),
 * which covers every shape the decode variant accepts (its workspace is at
 * most 16 MiB, at 255 rows); a larger need returns DSA_ERR_UNSUPPORTED.
 * Nothing is allocated or freed. All calls on one GPU share that GPU's
 * array and it keeps the last call's partials: calls that may overlap on
 * one GPU (other streams, other host threads) race and must be serialised
 * by the caller.
 */
int32_t dsa_sparse_mla_decode_noalloc(const dsa_batch* batch, const dsa_cache* cache, const void* q,
                                      int32_t num_heads, const int32_t* idx, int32_t k, float softmax_scale,
                                      void* out, float* lse, void* stream);

/*
 * The whole decode step: Score -> Select (top-k) -> Attend, as one call on
 * one stream. The pages' problem statement: for every query row the indexer
 * scores one FP8 key per earlier token, the top k are kept, and MLA runs
 * over only those rows ("TokenSpeed Kimi K3.1", section "Integrating sparse
 * attention with the K3 stack", steps 2-4).
 *   q_idx, q_dtype, q_scale, w: the indexer query and head weights, as
 *            dsa_index_score takes them: bf16 [rows][32][128] (q_scale
 *            NULL), or E4M3 codes with a row scale each (DSA_Q_FP8: the
 *            FP8 index queries of "TokenSpeed Kimi K3.1", section "Reducing
 *            indexer overhead on AMD MI350X"; one MFMA term per product
 *            instead of the bf16 split's two); w bf16 [rows][32]
 *   q_mla    bf16 [rows][num_heads][576]              (as dsa_sparse_mla_decode)
 *   out      bf16 [rows][num_heads][512]; lse fp32 [rows][num_heads] or NULL
 *   idx_out  int32 [rows][k] or NULL: receives the selection.
 *   ws       workspace of dsa_workspace_size(DSA_WS_DECODE, rows, max_ctx, k, num_heads)
 *            (holds the fp32 scores, the selection and the attention partials).
 * Results are the same as dsa_index_score -> dsa_topk -> dsa_sparse_mla_decode
 * (the same selected set). Batches with max_ctx up to 40,960 store every
 * score and select with the top-k kernels; longer ones run the filtered
 * path (dsa_filter_threshold -> dsa_filter_score -> dsa_filter_select below):
 * the scorer keeps only scores at or above a sampled per-row threshold, so
 * the fp32 score rows never go to HBM and back. Either way attention reads
 * the selection's cache rows directly.
 */
int32_t dsa_decode(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                   const float* q_scale, const void* w, const void* q_mla, int32_t num_heads, int32_t k,
                   float softmax_scale, void* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * dsa_decode with scores filtered inside the scorer against a per-row
 * threshold the caller gives: the scorer keeps (score, position) of every
 * score at or above the row's threshold instead of storing every score, and
 * the k largest of those candidates are selected. The fused indexer of
 * "vLLM Day-0 Support for Kimi K3.1 Pro", section "Fused low-latency decode
 * for DSA layers", likewise hands an exact top-k select only what its
 * scorer keeps. A row whose candidates cannot decide the result (fewer than
 * k reach the threshold, or more than the buffers hold) is scored again in
 * full and selected over its whole row, so the selection is always exact.
 * A good threshold is any value a little below the row's k-th score (for
 * instance the same request's k-th score at the previous decode step).
 *   threshold  fp32 [rows], device: the scorer keeps every score >= it. Any
 *              value works, NaN and +-inf included: too high a threshold
 *              (fewer than k scores reach it) or too low (more candidates
 *              than the buffers hold) sends the row to the exact fallback,
 *              so idx, out and lse are those of dsa_decode whatever it is.
 * Other arguments and the workspace are dsa_decode's. Returns
 * DSA_ERR_UNSUPPORTED if a request would need more than 1,024 scoring
 * workgroups (contexts beyond about 64M tokens).
 */
int32_t dsa_decode_thresholded(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                               const float* q_scale, const void* w, const void* q_mla, int32_t num_heads, int32_t k,
                               float softmax_scale, const float* threshold, void* out, float* lse, int32_t* idx_out,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * The filtered path's three stages, one call each, on one stream and one
 * workspace (dsa_decode's: dsa_workspace_size(DSA_WS_DECODE, rows, max_ctx,
 * k, 16)), which carries each stage's results to the next; call them in
 * order with the same batch, cache, queries and k. Together they select
 * exactly what dsa_topk selects over dsa_index_score's scores ("vLLM Day-0
 * Support for Kimi K3.1 Pro", section "Fused low-latency decode for DSA
 * layers": a scorer that keeps candidates for an exact top-k select).
 *   dsa_filter_threshold  each row's visible length and candidate threshold:
 *       the caller's (threshold, fp32 [rows] on the device, any value as in
 *       dsa_decode_thresholded) or, with threshold NULL, sampled: 8,192 of
 *       the row's scores (128 whole pages spread over its context; 4,096
 *       scores from 64 pages past 32 rows) and a value a little below the
 *       sampled rank that leaves about 1.25k scores of the row above it;
 *       rows of at most 8,192 tokens keep every score.
 *   dsa_filter_score      every score at or above its row's threshold, as
 *       (score, position), into the workspace; nothing else is stored.
 *   dsa_filter_select     idx int32 [rows][k]: the k largest candidates of
 *       each row (the selection of dsa_topk, padding -1 included); a row its
 *       candidates cannot decide is scored again in full and selected over
 *       all of it.
 * q_idx, q_dtype, q_scale and w are dsa_decode's (bf16 or E4M3 queries). Returns
 * DSA_ERR_UNSUPPORTED if a request would need more than 1,024 scoring
 * workgroups (contexts beyond about 64M tokens).
 */
int32_t dsa_filter_threshold(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                             const float* q_scale, const void* w, int32_t k, const float* threshold, void* ws,
                             size_t ws_bytes, void* stream);
int32_t dsa_filter_score(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                         const float* q_scale, const void* w, int32_t k, void* ws, size_t ws_bytes, void* stream);
int32_t dsa_filter_select(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                          const float* q_scale, const void* w, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Decode context parallelism, simulated on one device. Under DCP, token p of
 * a request lives on shard p mod W of W devices; each shard scores and ranks
 * only its own tokens, the shards merge their candidates exactly, attend to
 * the winners they own, and combine the partial outputs by log-sum-exp
 * ("Kimi K3.1 Pro: Day-0 Inference and RL Support with SGLang and Miles", section "Decode: DSA with decode
 * context parallelism"; "vLLM Day-0 Support for Kimi K3.1 Pro", section "An
 * exact top-k merge with about 10x less traffic"; "TokenSpeed Kimi K3.1",
 * section "Sharding long contexts with decode context parallelism"). Here the
 * W shards are regions of one device's memory: these calls reproduce the
 * protocol's results, not its communication.
 *
 * dsa_dcp_topk: per row, each shard's top-k and best C candidates; the
 * cutoff is the k-th best of all W * C candidates; a shard whose C
 * candidates all rank above the cutoff adds its whole top-k; the k best of
 * that pool are written to idx. Ranking is dsa_topk's (score, then lower
 * position), so idx holds exactly dsa_topk's set.
 *   scores, ld, row_len, rows, k, idx  as for dsa_topk.
 *   W        shards, 2 <= W <= 64, rows * W <= 65535; C candidates per
 *            shard, 1 <= C <= k (the
 *            pages use C = 1.5 k / W: 384 for k = 2048, W = 8).
 *   resend   uint8 [rows][W]: 1 where shard w added its whole top-k. With
 *            fewer than k candidates in all (short rows) there is no cutoff
 *            and every shard that sent C candidates resends; a shard with
 *            fewer than C tokens sent all of them and never resends.
 *   ws       dsa_dcp_workspace_size(DSA_WS_DCP_TOPK, rows, ld, k, W, C) bytes.
 * Scores must be finite (-inf marks positions outside a candidate pool).
 */
int32_t dsa_dcp_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t rows, int32_t k, int32_t W,
                     int32_t C, int32_t* idx, uint8_t* resend, void* ws, size_t ws_bytes, void* stream);

/*
 * dsa_dcp_mla_decode: shard w runs dsa_sparse_mla_decode over the entries of
 * idx it owns (p mod W == w, the others skipped), giving a bf16 partial
 * output and its lse; the W partials are combined as
 *   L = log sum_w exp(lse_w),  out = sum_w exp(lse_w - L) out_w,
 * into out (bf16 [rows][16][512]) and lse (fp32 [rows][16], may be NULL).
 * Arguments as for dsa_sparse_mla_decode, plus W (2..64); rows * W at most 65535.
 *   ws  dsa_dcp_workspace_size(DSA_WS_DCP_MLA, rows, 0, k, W, 0) bytes.
 */
int32_t dsa_dcp_mla_decode(const dsa_batch* batch, const dsa_cache* cache, const void* q, int32_t num_heads,
                           const int32_t* idx, int32_t k, int32_t W, float softmax_scale, void* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of the DCP entry points (ld is unused for DSA_WS_DCP_MLA, C
 * for DSA_WS_DCP_MLA). */
size_t dsa_dcp_workspace_size(int32_t kind, int32_t rows, int64_t ld, int32_t k, int32_t W, int32_t C);

/* Workspace bytes an entry point needs (0 if it needs none). For DSA_WS_TOPK,
 * `max_ctx` is the longest row_len. Returns 0 and no error for an unknown kind. */
size_t dsa_workspace_size(int32_t kind, int32_t rows, int64_t max_ctx, int32_t k, int32_t num_heads);

/* Text of a status code (static storage). */
const char* dsa_status_string(int32_t status);

/* Message of the last DSA_ERR_HIP or argument error on the calling host thread
 * (thread-local static storage; empty if none). */
const char* dsa_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
