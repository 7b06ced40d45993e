// Exact top-k selection: sampled threshold, one filtering pass, radix select
// over the survivors.
//
// "TokenSpeed Kimi K3.1", step 3: the 2,048 highest-scoring positions are
// kept per query row; section "Reducing indexer overhead on AMD MI350X": a
// row is spread over several workgroups, because one workgroup per row
// would leave most of the 256 compute units idle at 4-16 decode rows.
//
// Every element is ranked by the 64-bit composite (ordered score key << 32) |
// ~position, which is unique: larger score first, then lower position. The
// top k composites are a unique set, the same on every run.
//
// Kernels, all on one stream:
//  sample  one workgroup per row reads 8,192 scores in 64 evenly spaced runs
//          of 128 and takes a threshold T a little below the score rank that
//          should leave ~1.25k elements of the row above it (rows of at most
//          kTakeAll elements keep everything); it also zeroes the row's
//          candidate counter and, in the fused decode, writes the row's
//          visible length;
//  filter  several workgroups per row stream the row once with 16-byte loads
//          and compact every (key, position) with key >= T into the row's
//          candidate buffer: LDS lists, one global atomic per workgroup;
//  final   one workgroup per row radix-selects the k largest composites
//          among the candidates (in LDS when they fit). The answer is exact
//          whenever at least k candidates were collected, because every
//          element of the top k is then >= T; if fewer than k or more than
//          the buffer holds arrived, the workgroup selects over the whole row
//          instead. The sample only decides the speed, never the result.
#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int kT = 256;           // threads per workgroup
static constexpr int kSample = 8192;     // scores sampled per row
static constexpr int kRuns = 64;         // ... in this many evenly spaced runs
static constexpr int kRunLen = kSample / kRuns;
static constexpr int kTakeAll = 8192;    // rows up to this length keep every element
static constexpr int kListLds = 4096;    // candidates a filter workgroup buffers in LDS
static constexpr int kFinalLds = 8192;   // candidates the final kernel holds in LDS

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Candidate slots per row: 64 MB spread over the rows, clamped to
// [8192, 32768] (at least kTakeAll, well above the ~1.25k + margin that a
// sampled threshold leaves).
static int32_t cand_cap(int rows) {
  int64_t c = (int64_t)(64ll << 20) / 8 / (rows > 0 ? rows : 1);
  if (c > 32768) c = 32768;
  if (c < 8192) c = 8192;
  return (int32_t)(c / 64 * 64);
}

size_t topk_ws_bytes(int rows, int64_t max_len) {
  (void)max_len;
  return align_up((size_t)rows * 4, 256) * 2 + align_up((size_t)rows * cand_cap(rows) * 8, 256);
}

TopkWs topk_ws_carve(void* ws, int rows, int64_t max_len) {
  (void)max_len;
  TopkWs w;
  char* p = static_cast<char*>(ws);
  w.thresh = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * 4, 256);
  w.ctr = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * 4, 256);
  w.cand = reinterpret_cast<uint2*>(p);
  w.cap = cand_cap(rows);
  return w;
}

// ------------------------------------------------------------------ helpers

// Append the predicated lanes of a wave to a counter (LDS or global); returns
// each predicated lane's slot. One atomic per wave.
DSA_DEV uint32_t wave_append(uint32_t* counter, bool pred) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return 0;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
  base = __shfl(base, leader);
  const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  return base + below;
}

// Exclusive prefix of small per-lane counts (0..31) over the wave, from five
// bit-sliced ballots (no LDS traffic); total is the wave sum.
DSA_DEV uint32_t wave_prefix_small(uint32_t cnt, uint32_t& total) {
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {
    const uint64_t m = __ballot((cnt >> bit) & 1u);
    pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << bit;
    tot += (uint32_t)__popcll(m) << bit;
  }
  total = tot;
  return pre;
}

// One atomic per wave reserves `total` consecutive slots; all lanes get the base.
DSA_DEV uint32_t wave_reserve(uint32_t* counter, uint32_t total) {
  uint32_t base = 0;
  if (total != 0) {
    if ((threadIdx.x & 63) == 0) base = atomicAdd(counter, total);
    base = __builtin_amdgcn_readfirstlane(base);
  }
  return base;
}

struct Thresh {
  int digit;       // the bin holding the need-th largest element
  uint32_t above;  // elements in bins strictly above it
  uint32_t at;     // elements in that bin
};

struct ScanLds {
  uint32_t wsum[kT / 64];
  uint32_t res[3];
};

// Thread t owns bins [8t, 8t+8) with counts c[]; need >= 1 and at most the
// total. Finds d with count(bins > d) < need <= count(bins >= d). Two barriers.
DSA_DEV Thresh block_threshold(const uint32_t (&c)[8], uint32_t need, ScanLds& s) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mine += c[i];
  uint32_t suf = mine;  // inclusive suffix sum over the wave's lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(suf, off);
    if (lane + off < 64) suf += v;
  }
  if (lane == 0) s.wsum[wave] = suf;
  if (t == 0) s.res[0] = s.res[1] = s.res[2] = 0;
  __syncthreads();
  uint32_t above = suf - mine;
  for (int w = wave + 1; w < kT / 64; ++w) above += s.wsum[w];
  if (above < need && need <= above + mine) {
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above < need && need <= above + c[i]) {
        s.res[0] = 8 * t + i;
        s.res[1] = above;
        s.res[2] = c[i];
      }
      above += c[i];
    }
  }
  __syncthreads();
  Thresh r{(int)s.res[0], s.res[1], s.res[2]};
  __syncthreads();
  return r;
}

// Bins of an 11-bit digit: thread t reads its eight counters.
DSA_DEV void load_bins(const uint32_t* hist, uint32_t (&c)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = hist[8 * threadIdx.x + i];
}

DSA_DEV uint64_t composite(uint32_t key, uint32_t pos) { return ((uint64_t)key << 32) | (uint64_t)(~pos); }

struct MinMaxLds {
  uint64_t lo[kT / 64];
  uint64_t hi[kT / 64];
};

// Workgroup-wide (min, max) of one value per thread; one barrier pair.
DSA_DEV void block_minmax(uint64_t& lo, uint64_t& hi, MinMaxLds& s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t a = __shfl_xor(lo, off), b = __shfl_xor(hi, off);
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  if (lane == 0) {
    s.lo[wave] = lo;
    s.hi[wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kT / 64; ++w) {
    lo = s.lo[w] < lo ? s.lo[w] : lo;
    hi = s.hi[w] > hi ? s.hi[w] : hi;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ sample

__global__ __launch_bounds__(kT) void topk_sample_kernel(const float* __restrict__ scores, int64_t ld,
                                                        int32_t* __restrict__ row_len, const int32_t* ctx_len,
                                                        int R, int k, TopkWs w) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ ScanLds scan;
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  int64_t n;
  if (ctx_len) {  // fused decode: derive and publish the visible length
    n = ctx_len[row / R] - R + row % R + 1;
    if (t == 0) row_len[row] = (int32_t)n;
  } else {
    n = row_len[row];
  }
  if (t == 0) w.ctr[row] = 0;
  if (n <= kTakeAll) {  // keep every element (also covers n <= k)
    if (t == 0) w.thresh[row] = 0u;
    return;
  }
  // Sample j (thread t takes j = t + 256 i) is element (j % 128) of run j / 128.
  const float* s = scores + (size_t)row * ld;
  uint32_t key[kSample / kT];
#pragma unroll
  for (int i = 0; i < kSample / kT; ++i) {
    const int j = t + kT * i;
    const int64_t start = (int64_t)(j / kRunLen) * (n - kRunLen) / (kRuns - 1);
    key[i] = ordered_key(s[start + j % kRunLen]);
  }
  // Rank m of the threshold among the samples: the sampled share of 1.25k,
  // plus 32 so that a sample short of the true k-th score stays very unlikely.
  const double share = (double)kSample / (double)n;
  uint32_t m = (uint32_t)(1.25 * k * share) + 32u;
  if (m > (uint32_t)kSample) m = kSample;
  // Two 11-bit radix steps on the keys: T is the lower edge of the 22-bit
  // prefix bin that holds the m-th largest sample.
  uint32_t prefix = 0;
  for (int step = 0; step < 2; ++step) {
    const int shift = step == 0 ? 21 : 10;
    for (int i = t; i < kHistBins; i += kT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSample / kT; ++i)
      if (step == 0 || (key[i] >> 21) == prefix) atomicAdd(&hist[(key[i] >> shift) & (kHistBins - 1)], 1u);
    __syncthreads();
    uint32_t c[8];
    load_bins(hist, c);
    const Thresh th = block_threshold(c, m, scan);
    m -= th.above;
    prefix = step == 0 ? (uint32_t)th.digit : (prefix << 11) | (uint32_t)th.digit;
  }
  if (t == 0) w.thresh[row] = prefix << 10;
}

// ------------------------------------------------------------------ filter

struct FilterLds {
  uint32_t cnt;
  uint32_t base;
  uint2 list[kListLds];
};

template <bool VEC>
__global__ __launch_bounds__(kT) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ row_len, int slice, int k,
                                                        TopkWs w) {
  __shared__ FilterLds L;
  const int t = threadIdx.x;
  const int row = blockIdx.y;
  const int64_t n = row_len[row];
  if (n <= k) return;  // the final kernel emits every position
  const int64_t s0 = (int64_t)blockIdx.x * slice;
  const int64_t s1 = s0 + slice < n ? s0 + slice : n;
  const uint32_t T = w.thresh[row];
  uint32_t* ctr = w.ctr + row;
  uint2* gcand = w.cand + (size_t)row * w.cap;
  const float* s = scores + (size_t)row * ld;
  if (t == 0) L.cnt = 0;
  __syncthreads();

  // Each lane classifies 16 scores per step into a bitmask; one LDS atomic
  // per wave reserves the slots (uniform trip counts).
  const int lane = t & 63, wave = t >> 6;
  for (int64_t base = s0; base < s1; base += 16 * kT) {
    const int64_t wbase = base + 1024 * wave + 4 * lane;  // element (q, e): wbase + 256 q + e
    float v[16];
    if (VEC) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t i = wbase + 256 * q;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (i < s1) x = *reinterpret_cast<const f32x4*>(s + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t i = wbase + 256 * (j >> 2) + (j & 3);
        v[j] = i < s1 ? s[i] : 0.f;
      }
    }
    uint32_t cmask = 0;
    uint32_t keys[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t i = wbase + 256 * (j >> 2) + (j & 3);
      keys[j] = ordered_key(v[j]);
      cmask |= (uint32_t)(i < s1 && keys[j] >= T) << j;
    }
    uint32_t tc;
    const uint32_t pc = wave_prefix_small((uint32_t)__popc(cmask), tc);
    const uint32_t bc = wave_reserve(&L.cnt, tc);
    uint32_t slot = bc + pc;
    while (cmask) {
      const int j = __builtin_ctz(cmask);
      cmask &= cmask - 1;
      const uint2 e = make_uint2(keys[j], (uint32_t)(wbase + 256 * (j >> 2) + (j & 3)));
      if (slot < (uint32_t)kListLds) {
        L.list[slot] = e;
      } else {  // LDS list full: straight to the row's buffer
        const uint32_t gs = atomicAdd(ctr, 1u);
        if (gs < (uint32_t)w.cap) gcand[gs] = e;
      }
      ++slot;
    }
  }
  __syncthreads();
  if (t == 0) {
    const uint32_t nc = L.cnt < (uint32_t)kListLds ? L.cnt : (uint32_t)kListLds;
    L.base = nc ? atomicAdd(ctr, nc) : 0;
    L.cnt = nc;
  }
  __syncthreads();
  for (uint32_t i = t; i < L.cnt; i += kT)
    if (L.base + i < (uint32_t)w.cap) gcand[L.base + i] = L.list[i];
}

// ------------------------------------------------------------------ final

static constexpr int kBinLds = 2048;  // threshold-bin elements kept for the last steps

struct FinalLds {
  ScanLds scan;
  MinMaxLds mm;
  uint32_t emitted;
  uint32_t nbin;
  uint32_t hist[kHistBins];
  uint64_t bin[kBinLds];
  uint2 elems[kFinalLds];
};

// Emit the positions of the k largest composites among `count` elements
// (comp_at(i) gives element i's composite).
//  1. The radix digits start below the bits every element shares (the
//     survivors of one row have close scores: their top bits would all fall
//     in one bin).
//  2. One 11-bit step finds the bin b holding the k-th largest; a second
//     pass emits everything above b and gathers b's elements into LDS.
//  3. Further 11-bit steps over the gathered elements resolve the rest
//     (without the gather, when b holds more than kBinLds elements).
template <class CompAt>
DSA_DEV void select_top(FinalLds& L, int64_t count, int k, int32_t* __restrict__ out, CompAt comp_at) {
  const int t = threadIdx.x;
  uint64_t lo = ~0ull, hi = 0;
  for (int64_t i = t; i < count; i += kT) {
    const uint64_t c = comp_at(i);
    lo = c < lo ? c : lo;
    hi = c > hi ? c : hi;
  }
  block_minmax(lo, hi, L.mm);
  if (t == 0) {
    L.emitted = 0;
    L.nbin = 0;
  }
  // the composites are distinct, so lo == hi only for a single element
  if (lo == hi) {
    if (t == 0) out[0] = (int32_t)~(uint32_t)hi;
    return;
  }
  int shift = 64 - __clzll((long long)(lo ^ hi));  // bits below the shared prefix
  uint64_t prefix = shift == 64 ? 0 : hi >> shift;
  uint32_t need = (uint32_t)k;

  // step over all elements
  int width = shift < 11 ? shift : 11;
  int lo_bit = shift - width;
  for (int i = t; i < kHistBins; i += kT) L.hist[i] = 0;
  __syncthreads();
  for (int64_t i = t; i < count; i += kT)
    atomicAdd(&L.hist[(comp_at(i) >> lo_bit) & ((1ull << width) - 1)], 1u);
  __syncthreads();
  uint32_t cnt[8];
  load_bins(L.hist, cnt);
  Thresh th = block_threshold(cnt, need, L.scan);
  const uint64_t b = (shift == 64 ? 0 : prefix << width) | (uint64_t)th.digit;  // top (64 - b_shift) bits
  const int b_shift = lo_bit;
  const bool gather = th.at <= (uint32_t)kBinLds;
  // emit everything above b; gather b
  for (int64_t base = 0; base < count; base += kT) {
    const int64_t i = base + t;
    uint64_t c = 0;
    bool above = false, at = false;
    if (i < count) {
      c = comp_at(i);
      above = (c >> b_shift) > b;
      at = gather && (c >> b_shift) == b;
    }
    const uint32_t slot = wave_append(&L.emitted, above);
    if (above) out[slot] = (int32_t)~(uint32_t)c;
    const uint32_t bslot = wave_append(&L.nbin, at);
    if (at) L.bin[bslot] = c;
  }
  __syncthreads();
  need -= th.above;
  const uint32_t emitted0 = th.above;
  if (th.at == need) {  // all of b is selected
    if (gather) {
      for (uint32_t i = t; i < th.at; i += kT) out[emitted0 + i] = (int32_t)~(uint32_t)L.bin[i];
    } else {
      if (t == 0) L.emitted = 0;
      __syncthreads();
      for (int64_t base = 0; base < count; base += kT) {
        const int64_t i = base + t;
        bool take = false;
        uint64_t c = 0;
        if (i < count) {
          c = comp_at(i);
          take = (c >> b_shift) == b;
        }
        const uint32_t slot = wave_append(&L.emitted, take);
        if (take) out[emitted0 + slot] = (int32_t)~(uint32_t)c;
      }
    }
    return;
  }
  // resolve within b: element j of the bin is bin_at(j)
  const int64_t nb = gather ? (int64_t)th.at : count;
  auto bin_at = [&](int64_t j) -> uint64_t { return gather ? L.bin[j] : comp_at(j); };
  prefix = b;
  shift = lo_bit;
  while (true) {
    width = shift < 11 ? shift : 11;
    lo_bit = shift - width;
    for (int i = t; i < kHistBins; i += kT) L.hist[i] = 0;
    __syncthreads();
    for (int64_t j = t; j < nb; j += kT) {
      const uint64_t c = bin_at(j);
      if ((c >> shift) == prefix) atomicAdd(&L.hist[(c >> lo_bit) & ((1ull << width) - 1)], 1u);
    }
    __syncthreads();
    load_bins(L.hist, cnt);
    th = block_threshold(cnt, need, L.scan);
    need -= th.above;
    prefix = (prefix << width) | (uint64_t)th.digit;
    shift = lo_bit;
    if (th.at == need || shift == 0) break;
  }
  if (t == 0) L.emitted = 0;
  __syncthreads();
  // elements of b whose top (64 - shift) bits are at least the resolved prefix
  for (int64_t base = 0; base < nb; base += kT) {
    const int64_t j = base + t;
    bool take = false;
    uint64_t c = 0;
    if (j < nb) {
      c = bin_at(j);
      take = (gather || (c >> b_shift) == b) && (c >> shift) >= prefix;
    }
    const uint32_t slot = wave_append(&L.emitted, take);
    if (take && emitted0 + slot < (uint32_t)k) out[emitted0 + slot] = (int32_t)~(uint32_t)c;
  }
}

// One workgroup per row (a kernel boundary orders the filter's writes before
// these reads; a device-scope fence per workgroup would write back each
// XCD's L2).
__global__ __launch_bounds__(kT) void topk_final_kernel(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ row_len, int k,
                                                       int32_t* __restrict__ idx, TopkWs w) {
  __shared__ FinalLds L;
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const int64_t n = row_len[row];
  int32_t* out = idx + (size_t)row * k;
  if (n <= k) {  // every visible position is selected; the rest is padding
    for (int64_t i = t; i < k; i += kT) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  const uint32_t count = w.ctr[row];
  const uint2* gcand = w.cand + (size_t)row * w.cap;
  if (count >= (uint32_t)k && count <= (uint32_t)w.cap) {
    if (count <= (uint32_t)kFinalLds) {
      for (uint32_t base = 0; base < count; base += 8 * kT) {  // eight loads in flight per lane
        uint2 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t i = base + t + j * kT;
          v[j] = i < count ? gcand[i] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t i = base + t + j * kT;
          if (i < count) L.elems[i] = v[j];
        }
      }
      __syncthreads();
      select_top(L, count, k, out, [&](int64_t i) { return composite(L.elems[i].x, L.elems[i].y); });
    } else {
      select_top(L, count, k, out, [&](int64_t i) {
        const uint2 e = gcand[i];
        return composite(e.x, e.y);
      });
    }
  } else {  // the sample missed: select over the whole row
    const float* s = scores + (size_t)row * ld;
    select_top(L, n, k, out, [&](int64_t i) { return composite(ordered_key(s[i]), (uint32_t)i); });
  }
}

// ------------------------------------------------------------------ launcher

static bool vec_ok(const float* scores, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(scores) % 16) == 0 && (ld % 4) == 0;
}

hipError_t launch_topk(const float* scores, int64_t ld, int32_t* row_len, int rows, int64_t max_len, int k,
                       int32_t* idx, const TopkWs& w, hipStream_t st, const int32_t* ctx_len, int R) {
  hipLaunchKernelGGL(topk_sample_kernel, dim3(rows), dim3(kT), 0, st, scores, ld, row_len, ctx_len, R, k, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Filter: enough workgroups to cover the GPU twice, at least 4096 scores each.
  int64_t want = (512 + rows - 1) / rows;
  const int64_t max_slices = (max_len + 4095) / 4096;
  if (want > max_slices) want = max_slices;
  if (want < 1) want = 1;
  int64_t slice = (max_len + want - 1) / want;
  slice = (slice + 4095) / 4096 * 4096;
  const int ns = (int)((max_len + slice - 1) / slice);
  if (vec_ok(scores, ld))
    hipLaunchKernelGGL(topk_filter_kernel<true>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len, (int)slice,
                       k, w);
  else
    hipLaunchKernelGGL(topk_filter_kernel<false>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len,
                       (int)slice, k, w);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_final_kernel, dim3(rows), dim3(kT), 0, st, scores, ld, row_len, k, idx, w);
  return hipGetLastError();
}

}  // namespace dsa
