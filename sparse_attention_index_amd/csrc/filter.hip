// Filtered decode: the sampling pass before the scorer and the selection
// after it.
//
// The scorer in filter mode (score.hip) keeps, per row, only the
// (score, position) pairs at or above the row's threshold, so that the fp32
// score row never travels to HBM and back ("vLLM Day-0 Support for Kimi K3.1
// Pro", section "Fused low-latency decode for DSA layers": a key-balanced
// scorer hands an exact top-k select only what it keeps). This file holds
//  * the sampling pass: each row's threshold from a sample of its own
//    scores, scored here with the scorer's arithmetic;
//  * the selection: the k largest candidates of each row, exact whenever no
//    scoring workgroup overflowed its region of the row's buffer and at
//    least k candidates arrived: the row's k-th score is then >= the
//    threshold, so every element of the top k was kept. A row that fails the
//    test is scored again in full by its selecting workgroup and selected
//    over the whole row, so the result never depends on the threshold.
#include "common.h"
#include "kernels.h"
#include "query.h"
#include "select.h"

namespace dsa {

static constexpr int kSamplePages = 128;             // pages sampled per row (8,192 keys)
static constexpr int kSampleKeys = kSamplePages * kBlock;
static_assert(kSampleKeys == kSampleBufKeys, "the workspace holds a row's samples");
static constexpr int kSampleThreads = 512;           // most waves (one per row) scoring sampled pages
static constexpr int kSelectThreads = 1024;          // threshold of a row from its samples
static constexpr int kCandLds = 16384;               // candidates a selecting workgroup holds in LDS ...
static constexpr int kCandLdsTbl = 8192;             // ... or this many, beside its request's page table
static constexpr int kTblLds = 16384;                // pages of that table (1,048,576 tokens)

// ------------------------------------------------------------------ one page, straight from HBM

// A row's query operands (the scorer's: a bf16 row split into two E4M3
// terms, or E4M3 codes as they are), and the scaled weights of the 16 heads
// each lane reduces, for one wave.
template <bool QFP8, bool KF4>
struct RowQuery {
  i32x8 A[QFP8 ? 1 : 2][2];
  float wv[16];
};

// The operands of a loaded query row (lane n holds head n's values and
// weight bits, both lane halves); the head's scale (the power of two of the
// split, or the row scale of E4M3 codes) goes into its weight.
template <bool QFP8, bool KF4>
DSA_DEV void finish_row_query(const QueryRaw<QFP8, KF4>& raw, uint32_t wbits, RowQuery<QFP8, KF4>& q) {
  const int g = (threadIdx.x & 63) >> 5;
  const float head_scale = finish_query(raw, q.A);
  // head h's weight times its scale sits in lanes h and h + 32
  const float ws = __uint_as_float(wbits << 16) * head_scale;
#pragma unroll
  for (int i = 0; i < 16; ++i) q.wv[i] = __shfl(ws, 8 * (i >> 2) + 4 * g + (i & 3));
}

template <bool QFP8, bool KF4>
DSA_DEV void row_query(const ScoreArgs& a, size_t row, RowQuery<QFP8, KF4>& q) {
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  QueryRaw<QFP8, KF4> raw;
  fetch_query<QFP8, KF4>(a, row, n, g, raw);
  finish_row_query<QFP8, KF4>(raw, a.w[row * kIdxHeads + n], q);
}

// B operands of the 64 keys of one page (keys 32h + n for lane n of each
// half: lane half g, step s holds dims 64g + 32s + [0, 32); MXFP4: the MX
// block 2g + s and its E8M0 scale) and the key scales.
template <bool KF4>
struct PageKeys {
  i32x8 b[2][2];
  int sb[2][2];
  float ks[2];
};

template <bool KF4>
DSA_DEV void load_page(const ScoreArgs& a, int32_t pid, PageKeys<KF4>& p) {
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const size_t key = (size_t)pid * kBlock + 32 * h + n;
    if constexpr (KF4) {
      const uint8_t* kp = a.key_fp4 + key * (kIdxDim / 2);
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(a.key_e8m0 + key * 4);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(kp + 16 * (2 * g + st));
        p.b[h][st] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        p.sb[h][st] = (int)((sw >> (8 * (2 * g + st))) & 0xffu);
      }
      p.ks[h] = 1.f;
    } else {
      const uint8_t* kp = a.key_fp8 + key * kIdxDim + 64 * g;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 lo4 = *reinterpret_cast<const u32x4*>(kp + 32 * st);
        const u32x4 hi4 = *reinterpret_cast<const u32x4*>(kp + 32 * st + 16);
        p.b[h][st] = i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                           (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        p.sb[h][st] = 127;
      }
      p.ks[h] = a.key_scale[key];
    }
  }
}

// Scores of keys 32h + n (v[h], in both lane halves): the scorer's MFMAs and
// head-weighted ReLU reduction.
template <bool QFP8, bool KF4>
DSA_DEV void score_page(const RowQuery<QFP8, KF4>& q, const PageKeys<KF4>& p, float (&v)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int t = 0; t < (QFP8 ? 1 : 2); ++t)
#pragma unroll
      for (int st = 0; st < 2; ++st)
        acc = KF4 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q.A[t][st], p.b[h][st], acc, 0, 4, 0, 127, 0,
                                                                   p.sb[h][st])
                  : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q.A[t][st], p.b[h][st], acc, 0, 0, 0, 0, 0, 0);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum = __builtin_fmaf(q.wv[i], relu(acc[i]), sum);
    v[h] = halves_sum_pair(sum, sum) * p.ks[h];
  }
}

// ------------------------------------------------------------------ sampling pass

// Two kernels. The first scores the sampled pages of every row of more than
// kTakeAll tokens: NSP whole pages (128, or 64 past 32 rows) evenly spaced
// over the `full` pages that every such row of the request sees in full (at
// least 128, so the sampled pages are distinct), sampled page j being page
// floor(j * full / NSP). With up to 8 rows per request, a workgroup takes
// PPW sampled pages of one request for all its rows, one wave per row: the
// waves load the same pages, so all but the first copy come from the CU's
// cache, and the pages' latency is spread over the workgroups (each wave
// splits its row's query once per workgroup); more rows take
// sample_score_rows_kernel below. The second takes
// each row's threshold from its samples (sample_select: a little below the
// sampled rank that leaves about 1.25k of the row's scores above it).
template <bool KF4, int NSP, int PPW, bool QFP8>
__global__ __launch_bounds__(kSampleThreads) void sample_score_kernel(ScoreArgs a, float* __restrict__ samp) {
  static_assert(NSP <= kSamplePages, "the workspace holds 128 sampled pages per row");
  constexpr int WPQ = NSP / PPW;  // workgroups per request
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, n = lane & 31;
  const int R = a.R, b = blockIdx.x / WPQ, j0 = (blockIdx.x % WPQ) * PPW;
  const int r = wave;  // this wave's row (one workgroup holds all R <= 8 rows)
  const int64_t L = a.ctx_len[b];
  if (L <= kTakeAll) return;  // no row of the request sees more (its last row sees L tokens)
  // the query row and head weights go out first: they depend on nothing, and
  // their latency then overlaps the chain ctx_len -> page ids -> keys
  QueryRaw<QFP8, KF4> qraw;
  fetch_query<QFP8, KF4>(a, (size_t)b * R + r, n, g, qraw);
  const uint32_t wbits = a.w[((size_t)b * R + r) * kIdxHeads + n];
  // pages every sampled row of the request sees in full: those of its first
  // row, and at least 128 (a row with more than kTakeAll tokens sees them)
  const int64_t first = (L - R + 1) / kBlock;
  const uint32_t full = (uint32_t)(first > kSamplePages ? first : kSamplePages);
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
  int32_t pid[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) pid[i] = table[(uint32_t)((uint64_t)(j0 + i) * full / NSP)];
  PageKeys<KF4> pk[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) load_page<KF4>(a, pid[i], pk[i]);
  const size_t row = (size_t)b * R + r;
  if (L - R + r + 1 <= kTakeAll) return;  // this row keeps every score
  hold_query(qraw);
  RowQuery<QFP8, KF4> q;
  finish_row_query<QFP8, KF4>(qraw, wbits, q);
  float* out = samp + row * kSampleKeys;
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    float v[2];
    score_page<QFP8, KF4>(q, pk[i], v);
    if (g == 0) {
      out[(j0 + i) * kBlock + n] = v[0];
      out[(j0 + i) * kBlock + 32 + n] = v[1];
    }
  }
}

// Past 8 rows per request: a workgroup stages kRowPages sampled pages of one
// request in LDS once (each thread copies one 16-byte chunk of each page's
// keys and one scale word, into the scorer's swizzled layout) and scores
// them for 8 of the request's rows, one wave per row (workgroup row y of the
// grid takes rows 8y .. 8y + 7), one page at a time from LDS: a sampled page
// then crosses from L2 once per 8 rows rather than once per row.
static constexpr int kRowPages = 8;

template <bool KF4>
DSA_DEV int staged_chunk_off(int key, int j) {  // LDS offset of 16-byte chunk j of a staged key
  return KF4 ? key * (kIdxDim / 2) + ((j ^ ((key >> 2) & 3)) << 4) : key * kIdxDim + ((j ^ ((key >> 1) & 7)) << 4);
}

template <bool KF4>
DSA_DEV void lds_page(const uint8_t* keys, const uint32_t* ks, PageKeys<KF4>& p) {
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key = 32 * h + n;
    if constexpr (KF4) {
      const uint32_t sw = ks[key];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(keys + staged_chunk_off<true>(key, 2 * g + st));
        p.b[h][st] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        p.sb[h][st] = (int)((sw >> (8 * (2 * g + st))) & 0xffu);
      }
      p.ks[h] = 1.f;
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 lo4 = *reinterpret_cast<const u32x4*>(keys + staged_chunk_off<false>(key, 4 * g + 2 * st));
        const u32x4 hi4 = *reinterpret_cast<const u32x4*>(keys + staged_chunk_off<false>(key, 4 * g + 2 * st + 1));
        p.b[h][st] = i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                           (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        p.sb[h][st] = 127;
      }
      p.ks[h] = __uint_as_float(ks[key]);
    }
  }
}

template <bool KF4, int NSP, bool QFP8>
__global__ __launch_bounds__(kSampleThreads) void sample_score_rows_kernel(ScoreArgs a, float* __restrict__ samp) {
  static_assert(NSP <= kSamplePages && NSP % kRowPages == 0, "whole groups of the sampled pages");
  constexpr int WPQ = NSP / kRowPages;                     // workgroups per request and row group
  constexpr int KB = KF4 ? kBlock * kIdxDim / 2 : kBlock * kIdxDim;  // key bytes of a page
  constexpr int NCH = KB / 16;                             // 16-byte chunks of a page (512 or 256)
  static_assert(NCH <= kSampleThreads, "one chunk per thread and page");
  __shared__ __attribute__((aligned(16))) uint8_t keys_s[kRowPages][KB];
  __shared__ uint32_t ks_s[kRowPages][kBlock];  // fp32 key scales, or 4 E8M0 per key
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, n = lane & 31;
  const int R = a.R, b = blockIdx.x / WPQ, j0 = (blockIdx.x % WPQ) * kRowPages;
  const int r = (int)blockIdx.y * (kSampleThreads / 64) + wave;  // this wave's row
  const int64_t L = a.ctx_len[b];
  if (L <= kTakeAll) return;  // the whole workgroup: no row of the request sees more
  const bool has_row = r < R;  // the last row group may have spare waves
  QueryRaw<QFP8, KF4> qraw;
  fetch_query<QFP8, KF4>(a, (size_t)b * R + (has_row ? r : 0), n, g, qraw);
  const uint32_t wbits = a.w[((size_t)b * R + (has_row ? r : 0)) * kIdxHeads + n];
  const int64_t first = (L - R + 1) / kBlock;
  const uint32_t full = (uint32_t)(first > kSamplePages ? first : kSamplePages);
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
  // stage the workgroup's pages: every load first, then the LDS writes
  u32x4 ch[kRowPages];
  uint32_t sc[kRowPages];
  const int tc = t < NCH ? t : 0;  // threads past a page's chunks re-read chunk 0 and write nothing
#pragma unroll
  for (int i = 0; i < kRowPages; ++i) {
    const size_t pid = (uint32_t)table[(uint32_t)((uint64_t)(j0 + i) * full / NSP)];
    ch[i] = *reinterpret_cast<const u32x4*>((KF4 ? a.key_fp4 : a.key_fp8) + pid * KB + 16 * tc);
    sc[i] = KF4 ? reinterpret_cast<const uint32_t*>(a.key_e8m0)[pid * kBlock + (t & 63)]
                : __float_as_uint(a.key_scale[pid * kBlock + (t & 63)]);
  }
#pragma unroll
  for (int i = 0; i < kRowPages; ++i) {
    if (t < NCH) {
      const int key = t / (KB / kBlock / 16), j = t % (KB / kBlock / 16);
      *reinterpret_cast<u32x4*>(&keys_s[i][staged_chunk_off<KF4>(key, j)]) = ch[i];
    }
    if (t < kBlock) ks_s[i][t] = sc[i];
  }
  __syncthreads();  // the pages are staged (every wave reaches this)
  if (!has_row || L - R + r + 1 <= kTakeAll) return;  // no row, or a row that keeps every score
  hold_query(qraw);
  RowQuery<QFP8, KF4> q;
  finish_row_query<QFP8, KF4>(qraw, wbits, q);
  float* out = samp + ((size_t)b * R + r) * kSampleKeys;
  for (int i = 0; i < kRowPages; ++i) {
    PageKeys<KF4> pk;
    lds_page<KF4>(keys_s[i], ks_s[i], pk);
    float v[2];
    score_page<QFP8, KF4>(q, pk, v);
    if (g == 0) {
      out[(j0 + i) * kBlock + n] = v[0];
      out[(j0 + i) * kBlock + 32 + n] = v[1];
    }
  }
}

// One workgroup per row: the row's visible length goes to row_len, and its
// threshold to thr: -inf for rows of at most kTakeAll tokens (every score is
// kept), the caller's with thr_in set, else the sampled one, written as the
// float a kept score must reach.
__global__ __launch_bounds__(kSelectThreads) void sample_select_kernel(const int32_t* __restrict__ ctx_len, int R,
                                                                        const float* __restrict__ samp, int ns, int k,
                                                                        const float* thr_in, float* thr,
                                                                        int32_t* row_len) {
  constexpr int NT = kSelectThreads;
  __shared__ uint32_t hist[kHistBins];
  __shared__ ScanLds<NT> scan;
  const int t = threadIdx.x, row = blockIdx.x;
  const int64_t vis = (int64_t)ctx_len[row / R] - R + row % R + 1;
  const int64_t nvis = vis > 0 ? vis : 0;
  if (t == 0) row_len[row] = (int32_t)nvis;
  if (thr_in) {
    if (t == 0) thr[row] = thr_in[row];
    return;
  }
  if (nvis <= kTakeAll) {
    if (t == 0) thr[row] = -INFINITY;
    return;
  }
  // ns samples: thread t holds samples t + NT i (i < ns / NT)
  const float* s = samp + (size_t)row * kSampleKeys;
  uint32_t raw[kSampleKeys / NT];
#pragma unroll
  for (int i = 0; i < kSampleKeys / NT; ++i) raw[i] = t + NT * i < ns ? __float_as_uint(s[t + NT * i]) : 0u;
  const uint32_t T = sample_select<NT, kSampleKeys>(raw, nvis, k, hist, scan, ns);
  if (t == 0) thr[row] = key_threshold_float(T);
}

// ------------------------------------------------------------------ selection

static_assert(kTF == kMaxFilterWg, "one selecting thread per scoring workgroup slot");

struct CandLds {
  SelectLds s;
  uint32_t off[kMaxFilterWg + 1];  // each workgroup region's first candidate in the row's run; the total last
  uint32_t wsum[kTF / 64];
  uint32_t wmax[kTF / 64];
  union {
    uint2 elems[kCandLds];
    struct {
      uint2 elems[kCandLdsTbl];  // the same storage as elems above
      int32_t page[kTblLds];     // the request's page table: positions become cache rows as they are emitted
    } tbl;
  } u;
};
static_assert(sizeof(CandLds) <= 160 * 1024, "one selecting workgroup per CU");

// One workgroup per row. a: the scorer's arguments (the fallback writes the
// row's scores to a.scores); G: the scorer's workgroups per row group, split
// over the B requests as the scorer split them; compact: [rows][a.cap] room
// for a row's candidates past what LDS holds.
template <bool KF4, bool QFP8>
__global__ __launch_bounds__(kTF) void candidate_select_kernel(ScoreArgs a, int B, int G, const float* thr,
                                                               const int32_t* __restrict__ row_len, uint2* compact,
                                                               int k, int32_t* __restrict__ idx, SlotOut so) {
  __shared__ CandLds L;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = blockIdx.x, R = a.R;
  // every workgroup slot's count is loaded before the split is known (slots
  // past it hold stale values and are ignored)
  const uint32_t c_all = a.cand_count[(size_t)row * kMaxFilterWg + t];
  const int64_t n = row_len[row];  // published by the sampling pass
  // every candidate v has v >= thr, so its key is >= ordered_key(thr)
  const uint32_t T = ordered_key(thr[row]);
  int32_t* out = idx + (size_t)row * k;
  if (n <= k) {  // every visible position is selected; the rest is padding
    emit_all_positions(row, R, n, k, out, so);
    return;
  }
  const int npages = (int)((n + kBlock - 1) / kBlock);
  // with cache rows asked for, the request's page table is staged in LDS
  // if the candidates leave room for it (copied straight into LDS beside the
  // gather, so its latency overlaps the gather's); else the rows are looked
  // up after the selection
  constexpr int kTblPer = kTblLds / kTF;
  const bool tbl_fits = so.slots && npages <= kTblLds && npages <= so.max_blocks;
  // the scoring workgroups of this row's request, as the scorer split them
  const WgRange wr = wg_range(a.ctx_len, B, G, 0, row / R);
  const int nw = wr.count;  // <= kMaxFilterWg (checked by the host)
  const uint32_t sub = (uint32_t)(a.cap / nw);
  const uint32_t c = t < nw ? c_all : 0u;
  const uint32_t incl = wave_incl_sum(c);
  if (lane == 63) L.wsum[wave] = incl;
  const int bad = __syncthreads_or(c > sub);
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTF / 64; ++w) {
    const uint32_t x = L.wsum[w];
    before += w < wave ? x : 0u;
    total += x;
  }
  if (t < nw) L.off[t] = before + incl - c;
  if (t == 0) L.off[nw] = total;
  __syncthreads();
  const uint2* regions = a.cand + (size_t)row * a.cap;
  bool slots_done = false;
  if (!bad && total >= (uint32_t)k) {
    // gather: wave w copies the regions w, w + 16, ..., sixteen at a time
    // (the first 64 candidates of each, one load per lane: a single round
    // trip for up to 256 regions), into LDS when they fit, else into the
    // row's compact run; and finds the largest key
    const bool in_lds = total <= (uint32_t)kCandLds;
    const bool with_tbl = tbl_fits && total <= (uint32_t)kCandLdsTbl;
    uint2* const run = compact + (size_t)row * a.cap;
    constexpr int kBatch = 16;
    uint32_t kmax = 0;
    // dst: LDS or the compact run (the branch on in_lds is uniform, so each
    // copy loop stores to one kind of memory only)
    auto gather = [&](uint2* dst) {
      for (int r0 = wave; r0 < nw; r0 += kBatch * (kTF / 64)) {
        // Every lane loads (no branch around the loads, so that all sixteen
        // are in flight at once): lanes past a region's count re-read its
        // slot 0, regions past the last re-read region 0's (in bounds: a
        // region's count is at most sub here).
        uint2 v[kBatch];
        uint32_t o[kBatch], cr[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int r = r0 + u * (kTF / 64);
          o[u] = r < nw ? L.off[r] : 0u;
          cr[u] = r < nw ? L.off[r + 1] - o[u] : 0u;
          const uint32_t j = (uint32_t)lane < cr[u] ? (uint32_t)lane : 0u;
          v[u] = regions[(size_t)(r < nw ? r : 0) * sub + j];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if ((uint32_t)lane < cr[u]) {
            dst[o[u] + lane] = v[u];
            kmax = max(kmax, v[u].x);
          }
        }
        // regions of more than 64 candidates: the rest, one pass per 64
        // (unrolled: o and cr stay in registers)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int r = r0 + u * (kTF / 64);
          for (uint32_t j = 64 + lane; j < cr[u]; j += 64) {
            const uint2 x = regions[(size_t)r * sub + j];
            dst[o[u] + j] = x;
            kmax = max(kmax, x.x);
          }
        }
      }
    };
    if (with_tbl) {
      // entry (16 i + w) 64 + lane of the table for lane `lane` of wave w,
      // copy i (entries past the request's pages re-read entry 0); issued
      // just before the gather's loads, so waiting for those waits for these
      const int32_t* table = so.block_table + (size_t)(row / R) * so.max_blocks;
#pragma unroll
      for (int i = 0; i < kTblPer; ++i) {
        const int base = (kTF / 64 * i + wave) * 64;
        copy4_to_lds(table + (base + lane < npages ? base + lane : 0), &L.u.tbl.page[base]);
      }
    }
    // Few regions (a request's rows spread over at most 8 scoring
    // workgroups, as in a prefill chunk): each region gets a group of waves,
    // four loads in flight per lane, instead of one wave walking it 64 at a
    // time.
    auto gather_grouped = [&](uint2* dst) {
      const int wpr = (kTF / 64) / nw;  // waves per region (>= 2)
      const int r = wave / wpr;         // uniform
      if (r < nw) {
        const uint32_t o = L.off[r], c = L.off[r + 1] - o;  // c <= sub here
        const uint32_t step = 64u * (uint32_t)wpr;
        for (uint32_t j0 = (uint32_t)(wave % wpr) * 64u; j0 < c; j0 += 4u * step) {
          uint2 x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {  // clamped: slot 0 of the region exists (c >= 1)
            const uint32_t j = j0 + q * step + lane;
            x[q] = regions[(size_t)r * sub + (j < c ? j : 0u)];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t j = j0 + q * step + lane;
            if (j < c) {
              dst[o + j] = x[q];
              kmax = max(kmax, x[q].x);
            }
          }
        }
      }
    };
    if (2 * nw <= kTF / 64) {
      if (in_lds) gather_grouped(L.u.elems);
      else gather_grouped(run);
    } else if (in_lds) {
      gather(L.u.elems);
    } else {
      gather(run);
    }
    if (with_tbl) wait_vmcnt<0>();  // the table copies have landed (the barrier below publishes them)
    const uint32_t wm = wave_max32(kmax);
    if (lane == 0) L.wmax[wave] = wm;
    if (!in_lds) __threadfence();  // the compact run is read back by the whole workgroup
    __syncthreads();
    kmax = wave_max32(lane < kTF / 64 ? L.wmax[lane] : 0u);
    const uint64_t lo = (uint64_t)T << 32, hi = ((uint64_t)kmax << 32) | 0xffffffffull;
    const Emit emit{out, with_tbl ? so.slots + (size_t)row * k : nullptr, L.u.tbl.page};
    slots_done = with_tbl;
    // a row that keeps every score (threshold -inf) has no useful lower
    // bound: select_top then finds the extremes itself (a bound at -inf would
    // put every candidate in the first radix step's top bin)
    const bool bounded = T > ordered_key(-INFINITY);
    if (in_lds)
      select_top(L.s, total, k, emit, [&](int64_t i) { return composite(L.u.elems[i].x, L.u.elems[i].y); },
                 bounded, lo, hi);
    else
      select_top(L.s, total, k, emit, [&](int64_t i) { const uint2 e = run[i]; return composite(e.x, e.y); },
                 bounded, lo, hi);
  } else {
    // the candidates cannot decide this row: score it in full (waves take
    // pages w, w + 16, ...) and select over the whole row
    float* srow = a.scores + (size_t)row * a.ld;
    const int32_t* table = a.block_table + (size_t)(row / R) * a.max_blocks;
    RowQuery<QFP8, KF4> q;
    row_query<QFP8, KF4>(a, (size_t)row, q);
    const int nl = lane & 31;
    for (int p = wave; p < npages; p += kTF / 64) {
      PageKeys<KF4> pk;
      load_page<KF4>(a, table[p], pk);
      float v[2];
      score_page<QFP8, KF4>(q, pk, v);
      if (lane < 32) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t pos = (int64_t)p * kBlock + 32 * h + nl;
          if (pos < n) srow[pos] = v[h];
        }
      }
    }
    __threadfence();  // the row is read back by the whole workgroup
    __syncthreads();
    const Emit emit{out, nullptr, nullptr};
    select_top(L.s, n, k, emit, [&](int64_t i) { return composite(ordered_key(srow[i]), (uint32_t)i); });
  }
  if (so.slots && !slots_done) {  // uniform
    __syncthreads();  // the selection is written (workgroup-visible)
    emit_slots(row, R, k, out, so);
  }
}

// ------------------------------------------------------------------ launchers

// Pages sampled per row: 128 (8,192 keys) for up to 32 rows, 64 beyond,
// where the sampling pass would otherwise cost more than the tighter
// threshold saves the selection.
static int sampled_pages(int rows) { return rows > 32 ? 64 : kSamplePages; }

template <bool KF4, int NSP, bool QFP8>
static void launch_sample_score(const ScoreArgs& a, int rows, float* samp, hipStream_t st) {
  constexpr int kWaves = kSampleThreads / 64;
  const int B = rows / a.R;
  if (a.R > kWaves)
    hipLaunchKernelGGL((sample_score_rows_kernel<KF4, NSP, QFP8>), dim3(B * (NSP / kRowPages), (a.R + kWaves - 1) / kWaves),
                       dim3(kSampleThreads), 0, st, a, samp);
  else
    hipLaunchKernelGGL((sample_score_kernel<KF4, NSP, 2, QFP8>), dim3(B * (NSP / 2)), dim3(64 * a.R), 0, st, a, samp);
}

template <bool KF4, bool QFP8>
static void launch_sample_score(const ScoreArgs& a, int rows, float* samp, hipStream_t st) {
  if (sampled_pages(rows) == kSamplePages) launch_sample_score<KF4, kSamplePages, QFP8>(a, rows, samp, st);
  else launch_sample_score<KF4, 64, QFP8>(a, rows, samp, st);
}

// E4M3 query codes arrive with their row scales (a.q_scale set); bf16
// queries without.
hipError_t launch_sample_threshold(const ScoreArgs& a, int rows, int k, const float* thr_in, float* samp, float* thr,
                                   int32_t* row_len, hipStream_t st) {
  if (!thr_in) {
    const bool q8 = a.q_scale != nullptr;
    if (a.key_fp4) {
      if (q8) launch_sample_score<true, true>(a, rows, samp, st);
      else launch_sample_score<true, false>(a, rows, samp, st);
    } else {
      if (q8) launch_sample_score<false, true>(a, rows, samp, st);
      else launch_sample_score<false, false>(a, rows, samp, st);
    }
  }
  hipLaunchKernelGGL(sample_select_kernel, dim3(rows), dim3(kSelectThreads), 0, st, a.ctx_len, a.R, samp,
                     sampled_pages(rows) * kBlock, k, thr_in, thr, row_len);
  return hipGetLastError();
}

template <bool KF4, bool QFP8>
static void launch_candidate_select(const ScoreArgs& a, int B, int G, const float* thr, const int32_t* row_len,
                                    uint2* compact, int rows, int k, int32_t* idx, const SlotOut& so, hipStream_t st) {
  hipLaunchKernelGGL((candidate_select_kernel<KF4, QFP8>), dim3(rows), dim3(kTF), 0, st, a, B, G, thr, row_len,
                     compact, k, idx, so);
}

hipError_t launch_candidate_select(const ScoreArgs& a, int B, int G, const float* thr, const int32_t* row_len,
                                   uint2* compact, int rows, int k, int32_t* idx, const SlotOut& so, hipStream_t st) {
  const bool q8 = a.q_scale != nullptr;
  if (a.key_fp4) {
    if (q8) launch_candidate_select<true, true>(a, B, G, thr, row_len, compact, rows, k, idx, so, st);
    else launch_candidate_select<true, false>(a, B, G, thr, row_len, compact, rows, k, idx, so, st);
  } else {
    if (q8) launch_candidate_select<false, true>(a, B, G, thr, row_len, compact, rows, k, idx, so, st);
    else launch_candidate_select<false, false>(a, B, G, thr, row_len, compact, rows, k, idx, so, st);
  }
  return hipGetLastError();
}

}  // namespace dsa
