// C ABI of libdsa: host-side argument checks, workspace carving and launch
// sequencing. Declarations and semantics are in include/dsa.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "dsa.h"
#include "common.h"
#include "kernels.h"

using namespace dsa;

namespace {

thread_local char g_err[512];

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t check_batch(const dsa_batch* b) {
  if (!b) return fail(DSA_ERR_INVALID_ARG, "batch is null");
  if (b->num_requests < 1 || b->rows_per_request < 1)
    return fail(DSA_ERR_INVALID_ARG, "num_requests and rows_per_request must be >= 1");
  if (!b->ctx_len || !b->block_table) return fail(DSA_ERR_INVALID_ARG, "ctx_len or block_table is null");
  if (b->max_ctx < b->rows_per_request) return fail(DSA_ERR_INVALID_ARG, "max_ctx < rows_per_request");
  if ((int64_t)b->max_blocks * DSA_BLOCK < b->max_ctx)
    return fail(DSA_ERR_INVALID_ARG, "max_blocks * 64 < max_ctx");
  if ((int64_t)b->num_requests * b->rows_per_request > INT32_MAX / 2)
    return fail(DSA_ERR_UNSUPPORTED, "too many rows");
  return DSA_OK;
}

// The scorer's key planes for the cache's key format.
void set_keys(ScoreArgs& a, const dsa_cache* c) {
  const bool f4 = c->key_format == DSA_KEY_MXFP4;
  a.key_fp8 = f4 ? nullptr : c->key_fp8;
  a.key_scale = f4 ? nullptr : c->key_scale;
  a.key_fp4 = f4 ? c->key_fp4 : nullptr;
  a.key_e8m0 = f4 ? c->key_e8m0 : nullptr;
}

int32_t check_cache(const dsa_cache* c, bool keys, bool lat) {
  if (!c) return fail(DSA_ERR_INVALID_ARG, "cache is null");
  if (c->block_size != DSA_BLOCK) return fail(DSA_ERR_UNSUPPORTED, "block_size must be 64");
  if (c->num_blocks < 1) return fail(DSA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (keys && c->key_format != DSA_KEY_FP8 && c->key_format != DSA_KEY_MXFP4)
    return fail(DSA_ERR_UNSUPPORTED, "key_format must be DSA_KEY_FP8 or DSA_KEY_MXFP4");
  if (keys && c->key_format == DSA_KEY_MXFP4) {
    if (!c->key_fp4 || !c->key_e8m0) return fail(DSA_ERR_INVALID_ARG, "MXFP4 key planes are null");
    if (!aligned(c->key_fp4, 16) || !aligned(c->key_e8m0, 4))
      return fail(DSA_ERR_INVALID_ARG, "key_fp4 must be 16-byte and key_e8m0 4-byte aligned");
  }
  if (keys && c->key_format == DSA_KEY_FP8 && (!c->key_fp8 || !c->key_scale))
    return fail(DSA_ERR_INVALID_ARG, "key planes are null");
  if (lat && (!c->lat_fp8 || !c->lat_scale)) return fail(DSA_ERR_INVALID_ARG, "latent planes are null");
  if (keys && c->key_format == DSA_KEY_FP8 && !aligned(c->key_fp8, 16))
    return fail(DSA_ERR_INVALID_ARG, "key_fp8 must be 16-byte aligned");
  if (lat && !aligned(c->lat_fp8, 16)) return fail(DSA_ERR_INVALID_ARG, "lat_fp8 must be 16-byte aligned");
  return DSA_OK;
}

int32_t check_mla(int32_t num_heads, int32_t k, const void* q, const int32_t* idx, const void* out, bool need_idx) {
  if (num_heads != DSA_MLA_HEADS) return fail(DSA_ERR_UNSUPPORTED, "num_heads must be 16");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k must be in [1, 2048]");
  if (!q || (need_idx && !idx) || !out) return fail(DSA_ERR_INVALID_ARG, "q, idx or out is null");
  if (!aligned(q, 16)) return fail(DSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
  return DSA_OK;
}

int64_t decode_ld(int32_t max_ctx) { return ((int64_t)max_ctx + 63) / 64 * 64; }

// Candidate slots per row of the filtered decode, split into one region per
// scoring workgroup of the row's request: the sampled threshold leaves about
// 3k to 8k of a row's scores at long contexts (the selection holds up to
// 16,384 in LDS and selects from larger runs where they are); a workgroup
// that passes its region sends the row to the exact fallback.
int32_t filter_cap(int32_t rows) { return rows <= 128 ? 65536 : 32768; }

struct DecodeWs {
  float* scores;   // full scores: the stored path, and the filtered path's fallback
  int32_t* row_len;
  int32_t* idx;
  int32_t* slots;  // physical cache rows of the selection
  void* topk;
  void* mla;
  float* thr;       // filtered path: per-row score threshold
  float* samp;      // filtered path: [rows][kSampleBufKeys] sampled scores
  uint32_t* fcount; // filtered path: [rows][kMaxFilterWg] candidates per scoring workgroup
  uint2* fcand;     // filtered path: [rows][filter_cap] candidates, one region per scoring workgroup
  uint2* fcompact;  // filtered path: [rows][filter_cap] a row's candidates in one run (past LDS capacity)
};

size_t decode_ws_parts(int32_t rows, int64_t max_ctx, int32_t k, DecodeWs* out, void* base) {
  const int64_t ld = decode_ld((int32_t)max_ctx);
  const size_t sizes[] = {
      align256((size_t)rows * ld * sizeof(float)),                    // scores
      align256((size_t)rows * sizeof(int32_t)),                       // row_len
      align256((size_t)rows * k * sizeof(int32_t)),                   // idx
      align256((size_t)rows * k * sizeof(int32_t)),                   // slots
      align256(topk_ws_bytes(rows, ld)),                              // topk
      align256(mla_ws_bytes(rows, k, true)),                          // mla
      align256((size_t)rows * sizeof(float)),                         // thr
      align256((size_t)rows * kSampleBufKeys * sizeof(float)),        // samp
      align256((size_t)rows * kMaxFilterWg * sizeof(uint32_t)),       // fcount
      align256((size_t)rows * filter_cap(rows) * sizeof(uint2)),      // fcand
      align256((size_t)rows * filter_cap(rows) * sizeof(uint2)),      // fcompact
  };
  size_t total = 0;
  constexpr int kParts = sizeof(sizes) / sizeof(sizes[0]);
  char* part[kParts];
  for (int i = 0; i < kParts; ++i) {
    part[i] = static_cast<char*>(base) + total;
    total += sizes[i];
  }
  if (out) {
    out->scores = reinterpret_cast<float*>(part[0]);
    out->row_len = reinterpret_cast<int32_t*>(part[1]);
    out->idx = reinterpret_cast<int32_t*>(part[2]);
    out->slots = reinterpret_cast<int32_t*>(part[3]);
    out->topk = part[4];
    out->mla = sizes[5] ? part[5] : nullptr;
    out->thr = reinterpret_cast<float*>(part[6]);
    out->samp = reinterpret_cast<float*>(part[7]);
    out->fcount = reinterpret_cast<uint32_t*>(part[8]);
    out->fcand = reinterpret_cast<uint2*>(part[9]);
    out->fcompact = reinterpret_cast<uint2*>(part[10]);
  }
  return total;
}

int32_t run_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t rows, int32_t k, int32_t* idx,
                 void* ws, hipStream_t st) {
  const TopkWs w = topk_ws_carve(ws, rows, ld);
  return hip_status(launch_topk(scores, ld, const_cast<int32_t*>(row_len), rows, ld, k, idx, w, st), "topk");
}

int32_t run_mla(const dsa_batch* batch, const dsa_cache* cache, const void* q, const int32_t* idx, int32_t k,
                float softmax_scale, void* out, float* lse, void* ws, bool split, hipStream_t st,
                const int32_t* slots = nullptr) {
  MlaArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.idx = idx;
  a.slots = slots;
  a.lat_fp8 = cache->lat_fp8;
  a.lat_scale = cache->lat_scale;
  a.block_table = batch->block_table;
  a.max_blocks = batch->max_blocks;
  a.R = batch->rows_per_request;
  a.k = k;
  a.sm_scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  const int rows = batch->num_requests * batch->rows_per_request;
  return hip_status(launch_sparse_mla(a, rows, split, ws, st), "sparse mla");
}

}  // namespace

extern "C" {

// The indexer query's format: bf16 without row scales, or E4M3 codes with them.
static int32_t check_q_format(int32_t q_dtype, const float* q_scale) {
  if (q_dtype == DSA_Q_BF16) {
    if (q_scale) return fail(DSA_ERR_INVALID_ARG, "q_scale must be null for bf16 queries");
  } else if (q_dtype == DSA_Q_FP8) {
    if (!q_scale) return fail(DSA_ERR_INVALID_ARG, "q_scale is required for FP8 queries");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "q_dtype must be DSA_Q_BF16 or DSA_Q_FP8");
  }
  return DSA_OK;
}

int32_t dsa_index_score(const dsa_batch* batch, const dsa_cache* cache, const void* q, int32_t q_dtype,
                        const float* q_scale, const void* w, float* scores, int64_t ld, void* stream) {
  g_err[0] = 0;
  int32_t r = check_batch(batch);
  if (r) return r;
  if ((r = check_cache(cache, true, false))) return r;
  if (!q || !w || !scores) return fail(DSA_ERR_INVALID_ARG, "q, w or scores is null");
  if ((r = check_q_format(q_dtype, q_scale))) return r;
  if (ld < batch->max_ctx) return fail(DSA_ERR_INVALID_ARG, "ld < max_ctx");
  if (!aligned(q, 16)) return fail(DSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
  ScoreArgs a;
  a.q = q;
  a.q_scale = q_scale;
  a.w = static_cast<const uint16_t*>(w);
  set_keys(a, cache);
  a.ctx_len = batch->ctx_len;
  a.block_table = batch->block_table;
  a.max_blocks = batch->max_blocks;
  a.R = batch->rows_per_request;
  a.scores = scores;
  a.ld = ld;
  return hip_status(launch_index_score(a, batch->num_requests, batch->max_ctx, q_dtype == DSA_Q_FP8,
                                       static_cast<hipStream_t>(stream)),
                    "index score");
}

int32_t dsa_index_key_write(const dsa_batch* batch, const void* k, const float* ln_weight, const float* ln_bias,
                            float eps, uint8_t* key_fp8, float* key_scale, int32_t num_blocks, void* stream) {
  g_err[0] = 0;
  int32_t r = check_batch(batch);
  if (r) return r;
  if (!k || !ln_weight || !ln_bias || !key_fp8 || !key_scale)
    return fail(DSA_ERR_INVALID_ARG, "k, ln_weight, ln_bias, key_fp8 or key_scale is null");
  if (num_blocks < 1) return fail(DSA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (!(eps > 0.f) || !(eps < INFINITY)) return fail(DSA_ERR_INVALID_ARG, "eps must be positive and finite");
  if (!aligned(k, 4) || !aligned(ln_weight, 8) || !aligned(ln_bias, 8) || !aligned(key_fp8, 2))
    return fail(DSA_ERR_INVALID_ARG, "k, ln_weight, ln_bias or key_fp8 is misaligned");
  KeyWriteArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.ln_weight = ln_weight;
  a.ln_bias = ln_bias;
  a.eps = eps;
  a.ctx_len = batch->ctx_len;
  a.block_table = batch->block_table;
  a.max_blocks = batch->max_blocks;
  a.R = batch->rows_per_request;
  a.rows = batch->num_requests * batch->rows_per_request;
  a.key_fp8 = key_fp8;
  a.key_scale = key_scale;
  a.num_blocks = num_blocks;
  return hip_status(launch_index_key_write(a, static_cast<hipStream_t>(stream)), "index key write");
}

int32_t dsa_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t rows, int32_t k, int32_t* idx,
                 void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (rows < 0 || ld < 1) return fail(DSA_ERR_INVALID_ARG, "rows must be >= 0 and ld >= 1");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k must be in [1, 2048]");
  if (rows == 0) return DSA_OK;
  if (!scores || !row_len || !idx) return fail(DSA_ERR_INVALID_ARG, "scores, row_len or idx is null");
  if (ld > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "rows longer than 2^31 scores");
  const size_t need = dsa_workspace_size(DSA_WS_TOPK, rows, ld, k, 0);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "topk needs %zu workspace bytes", need);
  return run_topk(scores, ld, row_len, rows, k, idx, ws, static_cast<hipStream_t>(stream));
}

static int32_t mla_entry(bool split, const dsa_batch* batch, const dsa_cache* cache, const void* q,
                         int32_t num_heads, const int32_t* idx, int32_t k, float softmax_scale, void* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int32_t r = check_batch(batch);
  if (r) return r;
  if ((r = check_cache(cache, false, true))) return r;
  if ((r = check_mla(num_heads, k, q, idx, out, true))) return r;
  const int32_t rows = batch->num_requests * batch->rows_per_request;
  const size_t need = dsa_workspace_size(split ? DSA_WS_MLA_DECODE : DSA_WS_MLA_PREFILL, rows, 0, k, num_heads);
  if (need && (!ws || ws_bytes < need)) return fail(DSA_ERR_WORKSPACE, "sparse mla needs %zu workspace bytes", need);
  return run_mla(batch, cache, q, idx, k, softmax_scale, out, lse, ws, split, static_cast<hipStream_t>(stream));
}

int32_t dsa_sparse_mla_decode(const dsa_batch* batch, const dsa_cache* cache, const void* q, int32_t num_heads,
                              const int32_t* idx, int32_t k, float softmax_scale, void* out, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
  return mla_entry(true, batch, cache, q, num_heads, idx, k, softmax_scale, out, lse, ws, ws_bytes, stream);
}

int32_t dsa_sparse_mla_decode_noalloc(const dsa_batch* batch, const dsa_cache* cache, const void* q,
                                      int32_t num_heads, const int32_t* idx, int32_t k, float softmax_scale,
                                      void* out, float* lse, void* stream) {
  g_err[0] = 0;
  int32_t r = check_batch(batch);
  if (r) return r;
  if ((r = check_cache(cache, false, true))) return r;
  if ((r = check_mla(num_heads, k, q, idx, out, true))) return r;
  const int32_t rows = batch->num_requests * batch->rows_per_request;
  const size_t need = mla_ws_bytes(rows, k, true);
  if (need > mla_scratch_bytes())
    return fail(DSA_ERR_UNSUPPORTED, "%d rows need %zu scratch bytes, more than the library's %zu", rows, need,
                mla_scratch_bytes());
  void* ws = nullptr;
  if (need && (r = hip_status(mla_scratch(&ws), "scratch address"))) return r;
  return run_mla(batch, cache, q, idx, k, softmax_scale, out, lse, ws, true, static_cast<hipStream_t>(stream));
}

int32_t dsa_sparse_mla_prefill(const dsa_batch* batch, const dsa_cache* cache, const void* q, int32_t num_heads,
                               const int32_t* idx, int32_t k, float softmax_scale, void* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  return mla_entry(false, batch, cache, q, num_heads, idx, k, softmax_scale, out, lse, ws, ws_bytes, stream);
}

// dsa_decode takes the filtered path (scores filtered into candidates
// inside the scorer) for batches with max_ctx above this; shorter batches
// take the stored-score path, whose one-workgroup top-k of short rows needs
// no sampling pass.
static constexpr int kFilterMinCtx = 40960;

// The scorer's arguments for one batch (scores go to the workspace's score
// rows: the stored path's and the filtered path's fallback).
static ScoreArgs index_args(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, const float* q_scale,
                            const void* w, const DecodeWs& p) {
  ScoreArgs a;
  a.q = q_idx;
  a.q_scale = q_scale;  // set for E4M3 queries
  a.w = static_cast<const uint16_t*>(w);
  set_keys(a, cache);
  a.ctx_len = batch->ctx_len;
  a.block_table = batch->block_table;
  a.max_blocks = batch->max_blocks;
  a.R = batch->rows_per_request;
  a.scores = p.scores;
  a.ld = decode_ld(batch->max_ctx);
  return a;
}

// The filtered path's view of the same arguments, and its scorer grid.
struct Filter {
  ScoreArgs f;
  int grid;  // scoring workgroups per row group (split over the requests)
  bool fits; // no request has more than kMaxFilterWg of them
};

static Filter filter_of(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, const float* q_scale,
                        const void* w, const DecodeWs& p) {
  Filter F;
  const int32_t rows = batch->num_requests * batch->rows_per_request;
  F.f = index_args(batch, cache, q_idx, q_scale, w, p);
  F.f.thr = p.thr;
  F.f.cand = p.fcand;
  F.f.cand_count = p.fcount;
  F.f.cap = filter_cap(rows);
  const int B = batch->num_requests;
  F.grid = filter_grid(B, batch->rows_per_request, batch->max_ctx, cache->key_format == DSA_KEY_MXFP4,
                       q_scale != nullptr);
  F.fits = F.grid - B + 1 <= kMaxFilterWg;
  return F;
}

// The three stages of the filtered path.
// 1. each row's visible length and threshold (sampled, or the caller's)
static int32_t filter_threshold(const Filter& F, const DecodeWs& p, int32_t rows, int32_t k, const float* thr_in,
                                hipStream_t st) {
  return hip_status(launch_sample_threshold(F.f, rows, k, thr_in, p.samp, p.thr, p.row_len, st), "filter threshold");
}
// 2. score, keeping only the candidates at or above the threshold
static int32_t filter_score(const Filter& F, const dsa_batch* batch, hipStream_t st) {
  return hip_status(launch_index_score(F.f, batch->num_requests, batch->max_ctx, F.f.q_scale != nullptr, st),
                    "filter score");
}
// 3. exact selection from the candidates; a row they cannot decide is
//    scored again in full (into the score rows) and selected over all of it
static int32_t filter_select(const Filter& F, const dsa_batch* batch, const DecodeWs& p, int32_t rows, int32_t k,
                             int32_t* idx, const SlotOut& so, hipStream_t st) {
  return hip_status(launch_candidate_select(F.f, batch->num_requests, F.grid, p.thr, p.row_len, p.fcompact, rows, k,
                                            idx, so, st),
                    "filter select");
}

// Checks shared by the decode entry points: batch, cache, indexer query and
// the workspace; the workspace carved into p.
static int32_t decode_checks(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                             const float* q_scale, const void* w, int32_t k, bool lat, void* ws, size_t ws_bytes,
                             DecodeWs* p) {
  int32_t r = check_batch(batch);
  if (r) return r;
  if ((r = check_cache(cache, true, lat))) return r;
  if (!q_idx || !w) return fail(DSA_ERR_INVALID_ARG, "q_idx or w is null");
  if ((r = check_q_format(q_dtype, q_scale))) return r;
  if (!aligned(q_idx, 16)) return fail(DSA_ERR_INVALID_ARG, "q_idx must be 16-byte aligned");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k must be in [1, 2048]");
  const int32_t rows = batch->num_requests * batch->rows_per_request;
  const size_t need = dsa_workspace_size(DSA_WS_DECODE, rows, batch->max_ctx, k, DSA_MLA_HEADS);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "decode needs %zu workspace bytes", need);
  decode_ws_parts(rows, batch->max_ctx, k, p, ws);
  return DSA_OK;
}

// The decode step. thr_in (device, [rows]) set: the filtered path with the
// caller's thresholds, whatever max_ctx is.
static int32_t decode_impl(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                           const float* q_scale, const void* w, const void* q_mla, int32_t num_heads, int32_t k,
                           float softmax_scale,
                           const float* thr_in, void* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                           void* stream) {
  g_err[0] = 0;
  DecodeWs p;
  int32_t r = check_mla(num_heads, k, q_mla, idx_out, out, false);
  if (r) return r;
  if ((r = decode_checks(batch, cache, q_idx, q_dtype, q_scale, w, k, true, ws, ws_bytes, &p))) return r;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t rows = batch->num_requests * batch->rows_per_request;
  int32_t* idx = idx_out ? idx_out : p.idx;
  SlotOut so;
  so.slots = p.slots;
  so.block_table = batch->block_table;
  so.max_blocks = batch->max_blocks;
  const Filter F = filter_of(batch, cache, q_idx, q_scale, w, p);
  if (thr_in && !F.fits)
    return fail(DSA_ERR_UNSUPPORTED, "a request would need more than %d scoring workgroups", kMaxFilterWg);
  if (thr_in || (batch->max_ctx > kFilterMinCtx && F.fits)) {
    if ((r = filter_threshold(F, p, rows, k, thr_in, st))) return r;
    if ((r = filter_score(F, batch, st))) return r;
    if ((r = filter_select(F, batch, p, rows, k, idx, so, st))) return r;
  } else {
    const ScoreArgs a = index_args(batch, cache, q_idx, q_scale, w, p);
    const int64_t ld = a.ld;
    const TopkWs tw = topk_ws_carve(p.topk, rows, ld);
    // 1. score
    if ((r = hip_status(launch_index_score(a, batch->num_requests, batch->max_ctx, q_dtype == DSA_Q_FP8, st),
                        "decode score")))
      return r;
    // 2. select (the visible lengths are derived on the way), also writing the
    //    cache rows of the selection so that attention reads no block table
    if ((r = hip_status(launch_topk(p.scores, ld, p.row_len, rows, ld, k, idx, tw, st, batch->ctx_len,
                                    batch->rows_per_request, so),
                        "decode topk")))
      return r;
  }
  // 3. attend
  return run_mla(batch, cache, q_mla, idx, k, softmax_scale, out, lse, p.mla, true, st, p.slots);
}

// The filtered path's stages as entry points of their own (one workspace,
// the decode step's, carries their state from one call to the next).
static int32_t filter_stage(int stage, const dsa_batch* batch, const dsa_cache* cache, const void* q_idx,
                            int32_t q_dtype, const float* q_scale, const void* w, int32_t k, const float* thr_in,
                            int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  DecodeWs p;
  int32_t r = decode_checks(batch, cache, q_idx, q_dtype, q_scale, w, k, false, ws, ws_bytes, &p);
  if (r) return r;
  if (stage == 3 && !idx) return fail(DSA_ERR_INVALID_ARG, "idx is null");
  const Filter F = filter_of(batch, cache, q_idx, q_scale, w, p);
  if (!F.fits) return fail(DSA_ERR_UNSUPPORTED, "a request would need more than %d scoring workgroups", kMaxFilterWg);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t rows = batch->num_requests * batch->rows_per_request;
  if (stage == 1) return filter_threshold(F, p, rows, k, thr_in, st);
  if (stage == 2) return filter_score(F, batch, st);
  SlotOut so;  // no cache rows: the caller's attention resolves idx itself
  so.slots = nullptr;
  so.block_table = batch->block_table;
  so.max_blocks = batch->max_blocks;
  return filter_select(F, batch, p, rows, k, idx, so, st);
}

int32_t dsa_decode(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                   const float* q_scale, const void* w, const void* q_mla, int32_t num_heads, int32_t k,
                   float softmax_scale, void* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                   void* stream) {
  return decode_impl(batch, cache, q_idx, q_dtype, q_scale, w, q_mla, num_heads, k, softmax_scale, nullptr, out, lse,
                     idx_out, ws, ws_bytes, stream);
}

int32_t dsa_decode_thresholded(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                               const float* q_scale, const void* w, const void* q_mla, int32_t num_heads, int32_t k,
                               float softmax_scale, const float* threshold, void* out, float* lse, int32_t* idx_out,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!threshold) {
    g_err[0] = 0;
    return fail(DSA_ERR_INVALID_ARG, "threshold is null");
  }
  return decode_impl(batch, cache, q_idx, q_dtype, q_scale, w, q_mla, num_heads, k, softmax_scale, threshold, out,
                     lse, idx_out, ws, ws_bytes, stream);
}

int32_t dsa_filter_threshold(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                             const float* q_scale, const void* w, int32_t k, const float* threshold, void* ws,
                             size_t ws_bytes, void* stream) {
  return filter_stage(1, batch, cache, q_idx, q_dtype, q_scale, w, k, threshold, nullptr, ws, ws_bytes, stream);
}

int32_t dsa_filter_score(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                         const float* q_scale, const void* w, int32_t k, void* ws, size_t ws_bytes, void* stream) {
  return filter_stage(2, batch, cache, q_idx, q_dtype, q_scale, w, k, nullptr, nullptr, ws, ws_bytes, stream);
}

int32_t dsa_filter_select(const dsa_batch* batch, const dsa_cache* cache, const void* q_idx, int32_t q_dtype,
                          const float* q_scale, const void* w, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                          void* stream) {
  return filter_stage(3, batch, cache, q_idx, q_dtype, q_scale, w, k, nullptr, idx, ws, ws_bytes, stream);
}

size_t dsa_workspace_size(int32_t kind, int32_t rows, int64_t max_ctx, int32_t k, int32_t num_heads) {
  (void)num_heads;
  if (rows <= 0) return 0;
  switch (kind) {
    case DSA_WS_TOPK:
      return topk_ws_bytes(rows, max_ctx < 1 ? 1 : max_ctx);
    case DSA_WS_MLA_DECODE:
      return mla_ws_bytes(rows, k, true);
    case DSA_WS_MLA_PREFILL:
      return mla_ws_bytes(rows, k, false);
    case DSA_WS_DECODE:
      return decode_ws_parts(rows, max_ctx < 1 ? 1 : max_ctx, k, nullptr, nullptr);
    default:
      return 0;
  }
}

int32_t dsa_dcp_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t rows, int32_t k, int32_t W,
                     int32_t C, int32_t* idx, uint8_t* resend, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (rows < 0 || ld < 1) return fail(DSA_ERR_INVALID_ARG, "rows must be >= 0 and ld >= 1");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k must be in [1, 2048]");
  if (W < 2 || W > 64) return fail(DSA_ERR_UNSUPPORTED, "W must be in [2, 64]");
  if (C < 1 || C > k) return fail(DSA_ERR_INVALID_ARG, "C must be in [1, k]");
  if (rows == 0) return DSA_OK;
  if (!scores || !row_len || !idx || !resend) return fail(DSA_ERR_INVALID_ARG, "scores, row_len, idx or resend is null");
  if (ld > INT32_MAX) return fail(DSA_ERR_UNSUPPORTED, "rows longer than 2^31 scores");
  if ((int64_t)rows * W > 65535) return fail(DSA_ERR_UNSUPPORTED, "rows * W must be <= 65535");
  const size_t need = dsa_dcp_workspace_size(DSA_WS_DCP_TOPK, rows, ld, k, W, C);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "dcp topk needs %zu workspace bytes", need);
  return hip_status(launch_dcp_topk(scores, ld, row_len, rows, k, W, C, idx, resend, ws,
                                    static_cast<hipStream_t>(stream)),
                    "dcp topk");
}

int32_t dsa_dcp_mla_decode(const dsa_batch* batch, const dsa_cache* cache, const void* q, int32_t num_heads,
                           const int32_t* idx, int32_t k, int32_t W, float softmax_scale, void* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int32_t r = check_batch(batch);
  if (r) return r;
  if ((r = check_cache(cache, false, true))) return r;
  if ((r = check_mla(num_heads, k, q, idx, out, true))) return r;
  if (W < 2 || W > 64) return fail(DSA_ERR_UNSUPPORTED, "W must be in [2, 64]");
  const int32_t rows = batch->num_requests * batch->rows_per_request;
  if ((int64_t)rows * W > 65535) return fail(DSA_ERR_UNSUPPORTED, "rows * W must be <= 65535");
  const size_t need = dsa_dcp_workspace_size(DSA_WS_DCP_MLA, rows, 0, k, W, 0);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "dcp mla needs %zu workspace bytes", need);
  MlaArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.idx = idx;
  a.lat_fp8 = cache->lat_fp8;
  a.lat_scale = cache->lat_scale;
  a.block_table = batch->block_table;
  a.max_blocks = batch->max_blocks;
  a.R = batch->rows_per_request;
  a.k = k;
  a.sm_scale = softmax_scale;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  return hip_status(launch_dcp_mla(a, rows, W, ws, static_cast<hipStream_t>(stream)), "dcp mla");
}

size_t dsa_dcp_workspace_size(int32_t kind, int32_t rows, int64_t ld, int32_t k, int32_t W, int32_t C) {
  if (rows <= 0 || k < 1 || W < 1) return 0;
  switch (kind) {
    case DSA_WS_DCP_TOPK:
      return C < 1 ? 0 : dcp_topk_ws_bytes(rows, ld < 1 ? 1 : ld, k, W, C);
    case DSA_WS_DCP_MLA:
      return dcp_mla_ws_bytes(rows, k, W);
    default:
      return 0;
  }
}

const char* dsa_status_string(int32_t status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_err; }

int32_t dsa_version(void) { return 200; }

}  // extern "C"
