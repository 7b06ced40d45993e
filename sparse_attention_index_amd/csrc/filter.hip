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

static constexpr int kSamplePages = 32;              // pages sampled per row (2,048 keys)
static constexpr int kSampleKeys = kSamplePages * kBlock;
static constexpr int kSampleThreads = 512;           // 8 waves, 4 sampled pages each
static constexpr int kCandLds = 16384;               // candidates a selecting workgroup holds in LDS

// ------------------------------------------------------------------ one page, straight from HBM

// A row's query split (the scorer's), and the scaled weights of the 16 heads
// each lane reduces, for one wave.
template <bool KF4>
struct RowQuery {
  i32x8 A[2][2];
  float wv[16];
};

// The split of a loaded query row (lane n holds head n's values and
// weight bits, both lane halves).
template <bool KF4>
DSA_DEV void finish_row_query(const QueryRaw<false, KF4>& raw, uint32_t wbits, RowQuery<KF4>& q) {
  const int g = (threadIdx.x & 63) >> 5;
  const float head_scale = finish_query(raw, q.A);
  // head h's weight times its scale sits in lanes h and h + 32
  const float ws = __uint_as_float(wbits << 16) * head_scale;
#pragma unroll
  for (int i = 0; i < 16; ++i) q.wv[i] = __shfl(ws, 8 * (i >> 2) + 4 * g + (i & 3));
}

template <bool KF4>
DSA_DEV void row_query(const ScoreArgs& a, size_t row, RowQuery<KF4>& q) {
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  QueryRaw<false, KF4> raw;
  fetch_query<false, KF4>(a, row, n, g, raw);
  finish_row_query<KF4>(raw, a.w[row * kIdxHeads + n], q);
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
template <bool KF4>
DSA_DEV void score_page(const RowQuery<KF4>& q, const PageKeys<KF4>& p, float (&v)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int t = 0; t < 2; ++t)
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

// One workgroup per query row. The row's visible length n goes to row_len.
// A row of more than kTakeAll tokens scores 2,048 sampled keys -- 32 whole
// pages evenly spaced over the pages it sees in full -- and takes the
// top-k's sampled threshold over them (sample_select: a little below the
// sampled rank that leaves about 1.25k scores of the row above it), written
// as the float a kept score must reach. Shorter rows keep every score
// (-inf). With thr_in set the caller's thresholds are copied instead.
template <bool KF4>
__global__ __launch_bounds__(kSampleThreads) void sample_threshold_kernel(ScoreArgs a, int k, const float* thr_in,
                                                                         float* thr, int32_t* row_len) {
  constexpr int NT = kSampleThreads, NW = NT / 64, PPW = kSamplePages / NW;
  __shared__ float samp[kSampleKeys];
  __shared__ uint32_t hist[kHistBins];
  __shared__ ScanLds<NT> scan;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, n = lane & 31;
  const int row = blockIdx.x, R = a.R, b = row / R;
  // the query row and head weights go out first: they depend on nothing,
  // and their latency then overlaps the chain ctx_len -> page ids -> keys
  QueryRaw<false, KF4> qraw;
  fetch_query<false, KF4>(a, (size_t)row, n, g, qraw);
  const uint32_t wbits = a.w[(size_t)row * kIdxHeads + n];
  const int vis = a.ctx_len[b] - R + row % R + 1;
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
  const uint32_t full = (uint32_t)(nvis / kBlock);  // pages the row sees in full (> 128)
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
  // sampled page j (< 32) is full page floor(j * full / 32). The page ids,
  // then every key load of the wave's four pages, are issued before the
  // query is split, so the split overlaps their latency.
  int32_t pid[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) pid[i] = table[((uint32_t)(wave * PPW + i) * full) / kSamplePages];
  PageKeys<KF4> pk[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) load_page<KF4>(a, pid[i], pk[i]);
  hold_query(qraw);
  RowQuery<KF4> q;
  finish_row_query<KF4>(qraw, wbits, q);
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    float v[2];
    score_page<KF4>(q, pk[i], v);
    if (g == 0) {
      samp[(wave * PPW + i) * kBlock + n] = v[0];
      samp[(wave * PPW + i) * kBlock + 32 + n] = v[1];
    }
  }
  __syncthreads();
  uint32_t raw[kSample / NT];
#pragma unroll
  for (int i = 0; i < kSample / NT; ++i) raw[i] = t + NT * i < kSampleKeys ? __float_as_uint(samp[t + NT * i]) : 0u;
  const uint32_t T = sample_select<NT>(raw, nvis, k, hist, scan, kSampleKeys);
  if (t == 0) thr[row] = key_threshold_float(T);
}

// ------------------------------------------------------------------ selection

static_assert(kTF == kMaxFilterWg, "one selecting thread per scoring workgroup slot");

struct CandLds {
  SelectLds s;
  uint32_t off[kMaxFilterWg + 1];  // each workgroup region's first candidate in the row's run; the total last
  uint32_t wsum[kTF / 64];
  uint32_t wmax[kTF / 64];
  uint2 elems[kCandLds];
};

// One workgroup per row. a: the scorer's arguments (the fallback writes the
// row's scores to a.scores); G: the scorer's workgroups per row group, split
// over the B requests as the scorer split them; compact: [rows][a.cap] room
// for a row's candidates past what LDS holds.
template <bool KF4>
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
  const Emit emit{out, nullptr, nullptr};
  const uint2* regions = a.cand + (size_t)row * a.cap;
  if (!bad && total >= (uint32_t)k) {
    // gather: wave w copies the regions w, w + 16, ..., four regions' loads
    // in flight per lane, into LDS when they fit, else into the row's
    // compact run; and finds the largest key
    const bool in_lds = total <= (uint32_t)kCandLds;
    uint2* dst = in_lds ? L.elems : compact + (size_t)row * a.cap;
    uint32_t kmax = 0;
    for (int r0 = wave; r0 < nw; r0 += 4 * (kTF / 64)) {
      uint2 v[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u * (kTF / 64);
        const uint32_t cr = r < nw ? L.off[r + 1] - L.off[r] : 0u;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t j = lane + 64 * e;
          v[u][e] = j < cr ? regions[(size_t)r * sub + j] : make_uint2(0u, 0u);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u * (kTF / 64);
        const uint32_t o = r < nw ? L.off[r] : 0u;
        const uint32_t cr = r < nw ? L.off[r + 1] - o : 0u;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t j = lane + 64 * e;
          if (j < cr) {
            dst[o + j] = v[u][e];
            kmax = max(kmax, v[u][e].x);
          }
        }
        // regions of more than 128 candidates: the rest, one pass per 64
        for (uint32_t j = 128 + lane; j < cr; j += 64) {
          const uint2 x = regions[(size_t)r * sub + j];
          dst[o + j] = x;
          kmax = max(kmax, x.x);
        }
      }
    }
    const uint32_t wm = wave_max32(kmax);
    if (lane == 0) L.wmax[wave] = wm;
    if (!in_lds) __threadfence();  // the compact run is read back by the whole workgroup
    __syncthreads();
    kmax = wave_max32(lane < kTF / 64 ? L.wmax[lane] : 0u);
    const uint64_t lo = (uint64_t)T << 32, hi = ((uint64_t)kmax << 32) | 0xffffffffull;
    if (in_lds)
      select_top(L.s, total, k, emit, [&](int64_t i) { return composite(L.elems[i].x, L.elems[i].y); }, true, lo, hi);
    else
      select_top(L.s, total, k, emit, [&](int64_t i) { const uint2 e = dst[i]; return composite(e.x, e.y); }, true, lo,
                 hi);
  } else {
    // the candidates cannot decide this row: score it in full (waves take
    // pages w, w + 16, ...) and select over the whole row
    float* srow = a.scores + (size_t)row * a.ld;
    const int32_t* table = a.block_table + (size_t)(row / R) * a.max_blocks;
    RowQuery<KF4> q;
    row_query<KF4>(a, (size_t)row, q);
    const int npages = (int)((n + kBlock - 1) / kBlock);
    const int nl = lane & 31;
    for (int p = wave; p < npages; p += kTF / 64) {
      PageKeys<KF4> pk;
      load_page<KF4>(a, table[p], pk);
      float v[2];
      score_page<KF4>(q, pk, v);
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
    select_top(L.s, n, k, emit, [&](int64_t i) { return composite(ordered_key(srow[i]), (uint32_t)i); });
  }
  if (so.slots) {
    __syncthreads();  // the selection is written (workgroup-visible)
    emit_slots(row, R, k, out, so);
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_sample_threshold(const ScoreArgs& a, int rows, int k, const float* thr_in, float* thr,
                                   int32_t* row_len, hipStream_t st) {
  if (a.key_fp4)
    hipLaunchKernelGGL(sample_threshold_kernel<true>, dim3(rows), dim3(kSampleThreads), 0, st, a, k, thr_in, thr,
                       row_len);
  else
    hipLaunchKernelGGL(sample_threshold_kernel<false>, dim3(rows), dim3(kSampleThreads), 0, st, a, k, thr_in, thr,
                       row_len);
  return hipGetLastError();
}

hipError_t launch_candidate_select(const ScoreArgs& a, int B, int G, const float* thr, const int32_t* row_len,
                                   uint2* compact, int rows, int k, int32_t* idx, const SlotOut& so, hipStream_t st) {
  if (a.key_fp4)
    hipLaunchKernelGGL(candidate_select_kernel<true>, dim3(rows), dim3(kTF), 0, st, a, B, G, thr, row_len, compact, k,
                       idx, so);
  else
    hipLaunchKernelGGL(candidate_select_kernel<false>, dim3(rows), dim3(kTF), 0, st, a, B, G, thr, row_len, compact,
                       k, idx, so);
  return hipGetLastError();
}

}  // namespace dsa
