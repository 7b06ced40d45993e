// Launch interfaces of the gfx950 DSA kernels (internal to libdsa).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct ScoreArgs {
  const void* q;            // bf16 [rows][32][128] or E4M3 [rows][32][128]
  const float* q_scale;     // fp32 [rows] (E4M3 queries) or null
  const uint16_t* w;        // bf16 [rows][32]
  const uint8_t* key_fp8;   // [num_blocks][64][128] E4M3, or null with MXFP4 keys
  const float* key_scale;   // [num_blocks][64]
  const uint8_t* key_fp4 = nullptr;   // MXFP4 keys: [num_blocks][64][64] E2M1 pairs (even dim low nibble)
  const uint8_t* key_e8m0 = nullptr;  // MXFP4 keys: [num_blocks][64][4] E8M0 scale of dims 32j .. 32j+31
  const int32_t* ctx_len;   // [B]
  const int32_t* block_table;  // [B][max_blocks]
  int32_t max_blocks;
  int32_t R;                // rows per request
  float* scores;            // [rows][ld]
  int64_t ld;
  // Filtered decode: in place of the scores, every (ordered key, position)
  // whose score is >= the row's threshold goes to the scoring workgroup's
  // own region of the row's candidate buffer (cap / W slots from
  // j * (cap / W), for the request's W workgroups, j this one's index among
  // them), and each workgroup writes its true count per row to
  // cand_count[row * kMaxFilterWg + j] (also when it exceeds the region):
  // no atomics and nothing to clear.
  const float* thr = nullptr;     // [rows] score threshold (-inf keeps every score, NaN none)
  uint2* cand = nullptr;          // [rows][cap]
  uint32_t* cand_count = nullptr; // [rows][kMaxFilterWg]
  int32_t cap = 0;
};

// Scores every (row, visible token). B requests, max_ctx bounds ctx_len.
// With a.cand set the scores are filtered into candidates instead of
// stored. q_fp8: E4M3 query codes with row scales (a.q_scale), else bf16.
hipError_t launch_index_score(const ScoreArgs& a, int B, int max_ctx, bool q_fp8, hipStream_t st);
// Most scoring workgroups a request gets in the filtered decode.
constexpr int kMaxFilterWg = 1024;
// Workgroups per row group the scorer launches in the filtered decode for B
// requests of R rows of at most max_ctx tokens (bf16 or E4M3 queries); a
// request gets at most grid - B + 1 of them.
int filter_grid(int B, int R, int max_ctx, bool mxfp4, bool q_fp8);

// Sampling pass of the filtered decode: each row's visible length goes to
// row_len and its score threshold to thr (-inf for rows of at most 8,192
// tokens: everything is kept). A row of more tokens scores 8,192 sampled
// keys (128 whole pages evenly spaced over its full pages; 4,096 past 32
// rows) into samp[row] and takes the top-k's sampled threshold over them.
// With thr_in set, thr[row] = thr_in[row] and nothing is sampled.
constexpr int kSampleBufKeys = 8192;  // samp row stride
hipError_t launch_sample_threshold(const ScoreArgs& a, int rows, int k, const float* thr_in, float* samp, float* thr,
                                   int32_t* row_len, hipStream_t st);

struct TopkWs {
  uint32_t* cnt;   // [rows][64] survivors each slice workgroup found
  uint32_t* tmax;  // [rows][64] largest ordered key each slice workgroup saw
  uint32_t* thr;   // [rows] the row's sampled threshold (ordered key)
  uint2* cand;     // [rows][cap] (ordered key, position), one region per slice workgroup
  int32_t cap;
};

size_t topk_ws_bytes(int rows, int64_t max_len);
TopkWs topk_ws_carve(void* ws, int rows, int64_t max_len);

// Physical cache slots of a selection (page id * 64 + offset, -1 for
// padding), for rows laid out request-major with R rows per request.
struct SlotOut {
  int32_t* slots = nullptr;              // [rows][k], or null: not emitted
  const int32_t* block_table = nullptr;  // [B][max_blocks]
  int32_t max_blocks = 0;
};
// idx[row][0..k) = the k largest scores[row][0..row_len[row]) (positions,
// unordered; -1 padding for rows shorter than k). With ctx_len != null the
// visible lengths are derived (ctx_len[row / R] - R + row % R + 1) and also
// written to row_len; otherwise row_len is read. With so.slots set, the
// selection's physical slots are written too.
hipError_t launch_topk(const float* scores, int64_t ld, int32_t* row_len, int rows, int64_t max_len, int k,
                       int32_t* idx, const TopkWs& w, hipStream_t st, const int32_t* ctx_len = nullptr, int R = 1,
                       const SlotOut& so = SlotOut{});

// Filtered decode, selection (one workgroup per row): the k largest of the
// candidates the scorer kept for the row (a.cand / a.cand_count / a.cap; G
// the scorer's grid, whose split over the B requests is recomputed from
// ctx_len), exact whenever no workgroup region overflowed and at least k
// arrived; otherwise the row is scored again in full into a.scores (row
// stride a.ld) and selected over its whole row. Rows of at most k tokens
// take every position. idx and the slots (if asked for) are written for
// every row. compact: [rows][a.cap] room for a row's candidates past what
// LDS holds.
hipError_t launch_candidate_select(const ScoreArgs& a, int B, int G, const float* thr, const int32_t* row_len,
                                   uint2* compact, int rows, int k, int32_t* idx, const SlotOut& so, hipStream_t st);

struct MlaArgs {
  const uint16_t* q;        // bf16 [rows][16][576]
  const int32_t* idx;       // [rows][k]
  const int32_t* slots = nullptr;  // [rows][k] physical slots of idx, or null (then idx goes through block_table)
  const uint8_t* lat_fp8;   // [num_blocks][64][576]
  const float* lat_scale;   // [num_blocks][64]
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t R;
  int32_t k;
  float sm_scale;
  uint16_t* out;            // bf16 [rows][16][512]
  float* lse;               // [rows][16] or null
  int32_t q_rows = 0;               // nonzero: row r takes its query, request and block-table row
                                    // from row r % q_rows (several virtual shards of the same rows)
  const int32_t* nvalid = nullptr;  // [rows] or null: row r attends to idx[r][0 .. nvalid[r]) only
};

size_t mla_ws_bytes(int rows, int k, bool split);
// The library's own scratch for the no-allocation decode attention: its size
// and its device address on the current device (looked up once per device).
size_t mla_scratch_bytes();
hipError_t mla_scratch(void** out);

// Decode context parallelism over W virtual shards of one device.
size_t dcp_topk_ws_bytes(int rows, int64_t ld, int k, int W, int C);
hipError_t launch_dcp_topk(const float* scores, int64_t ld, const int32_t* row_len, int rows, int k, int W, int C,
                           int32_t* idx, uint8_t* resend, void* ws, hipStream_t st);
size_t dcp_mla_ws_bytes(int rows, int k, int W);
hipError_t launch_dcp_mla(const struct MlaArgs& a, int rows, int W, void* ws, hipStream_t st);
// split == true spreads each row's k positions over several workgroups and
// merges the partial results by log-sum-exp; false gives each row one workgroup.
hipError_t launch_sparse_mla(const MlaArgs& a, int rows, bool split, void* ws, hipStream_t st);

struct KeyWriteArgs {
  const uint16_t* k;         // bf16 [rows][128] new index keys
  const float* ln_weight;    // fp32 [128]
  const float* ln_bias;      // fp32 [128]
  float eps;
  const int32_t* ctx_len;    // [B]
  const int32_t* block_table;  // [B][max_blocks]
  int32_t max_blocks;
  int32_t R;                 // rows per request
  int32_t rows;              // B * R
  uint8_t* key_fp8;          // [num_blocks][64][128]
  float* key_scale;          // [num_blocks][64]
  int32_t num_blocks;
};
// LayerNorm + E4M3 absmax quantisation + paged write of each new row's key.
hipError_t launch_index_key_write(const KeyWriteArgs& a, hipStream_t st);

}  // namespace dsa
