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
// Two kernels on one stream:
//  filter  several workgroups per row. Each first derives the same threshold
//          T from the same sample of the row: 2,048 or 4,096 of its scores
//          in evenly spaced runs of 128; T sits a little
//          below the sampled rank that should leave ~1.25k elements of the
//          row above it (rows of at most kTakeAll elements keep everything).
//          It then streams its slice of the row once with 16-byte loads and
//          compacts every (key, position) with key >= T into LDS (overflow
//          straight to global), then into its own region of the row's
//          candidate buffer, with its count in its own slot: no global
//          atomics and nothing to clear first;
//  final   one workgroup per row gathers the slices' candidates into LDS
//          and radix-selects the k largest composites. The answer is exact
//          whenever at least k candidates were collected, because every
//          element of the top k is then >= T; if fewer than k or more than
//          fit arrived, the workgroup selects over the whole row instead.
//          The sample only decides the speed, never the result.
#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int kT = 256;           // threads per filter workgroup
static constexpr int kTF = 1024;         // threads per final workgroup
static constexpr int kSample = 4096;     // most scores sampled per row
static constexpr int kRunLen = 128;      // ... in evenly spaced runs of this length
static constexpr int kTakeAll = 8192;    // rows up to this length keep every element
static constexpr int kListLds = 4096;    // candidates a filter workgroup buffers in LDS
static constexpr int kFinalLds = 12288;  // candidates the final kernel holds in LDS
static constexpr int kMaxSlices = 64;    // filter workgroups per row at most

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Candidate slots per row: 64 MB spread over the rows, clamped to
// [8192, 32768] (at least kTakeAll, well above the ~1.25k + margin that a
// sampled threshold leaves); each filter slice of a row owns cap / slices.
static int32_t cand_cap(int rows) {
  int64_t c = (int64_t)(64ll << 20) / 8 / (rows > 0 ? rows : 1);
  if (c > 32768) c = 32768;
  if (c < 8192) c = 8192;
  return (int32_t)(c / 64 * 64);
}

size_t topk_ws_bytes(int rows, int64_t max_len) {
  (void)max_len;
  return align_up((size_t)rows * kMaxSlices * 4, 256) + align_up((size_t)rows * cand_cap(rows) * 8, 256);
}

TopkWs topk_ws_carve(void* ws, int rows, int64_t max_len) {
  (void)max_len;
  TopkWs w;
  char* p = static_cast<char*>(ws);
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * kMaxSlices * 4, 256);
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

template <int NT>
struct ScanLds {
  uint32_t wsum[NT / 64];
  uint32_t res[3];
};

// Thread t of NT owns bins [B t, B t + B) (B = 2048 / NT) with counts c[];
// need >= 1 and at most the total. Finds d with count(bins > d) < need <=
// count(bins >= d). Two barriers.
template <int NT>
DSA_DEV Thresh block_threshold(const uint32_t (&c)[kHistBins / NT], uint32_t need, ScanLds<NT>& s) {
  constexpr int B = kHistBins / NT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < B; ++i) mine += c[i];
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
  for (int w = wave + 1; w < NT / 64; ++w) above += s.wsum[w];
  if (above < need && need <= above + mine) {
#pragma unroll
    for (int i = B - 1; i >= 0; --i) {
      if (above < need && need <= above + c[i]) {
        s.res[0] = B * t + i;
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

// Bins of an 11-bit digit: thread t reads its counters.
template <int NT>
DSA_DEV void load_bins(const uint32_t* hist, uint32_t (&c)[kHistBins / NT]) {
  constexpr int B = kHistBins / NT;
#pragma unroll
  for (int i = 0; i < B; ++i) c[i] = hist[B * threadIdx.x + i];
}

DSA_DEV uint64_t composite(uint32_t key, uint32_t pos) { return ((uint64_t)key << 32) | (uint64_t)(~pos); }

template <int NT>
struct MinMaxLds {
  uint64_t lo[NT / 64];
  uint64_t hi[NT / 64];
};

// Workgroup-wide (min, max) of one value per thread; one barrier pair.
template <int NT>
DSA_DEV void block_minmax(uint64_t& lo, uint64_t& hi, MinMaxLds<NT>& s) {
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
  for (int w = 0; w < NT / 64; ++w) {
    lo = s.lo[w] < lo ? s.lo[w] : lo;
    hi = s.hi[w] > hi ? s.hi[w] : hi;
  }
  __syncthreads();
}

// ------------------------------------------------------------------ filter

// Visible length of a row: from row_len, or derived in the fused decode.
DSA_DEV int64_t visible_len(const int32_t* row_len, const int32_t* ctx_len, int R, int row) {
  return ctx_len ? (int64_t)ctx_len[row / R] - R + row % R + 1 : (int64_t)row_len[row];
}

struct FilterLds {
  ScanLds<kT> scan;
  uint32_t cnt;
  union {
    uint32_t hist[kHistBins];
    uint2 list[kListLds];
  } u;
};

// The ordered-key threshold of a row (the same in every workgroup of it).
DSA_DEV uint32_t sample_threshold(const float* __restrict__ s, int64_t n, int k, FilterLds& L) {
  const int t = threadIdx.x;
  if (n <= kTakeAll) return 0u;  // keep every element
  // ns samples (2048, or 4096 past 256K elements): sample j (thread t takes
  // j = t + 256 i) is element (j % 128) of run j / 128, the runs evenly
  // spaced over the row.
  const int ns = n > (1 << 18) ? 4096 : 2048;
  const int runs = ns / kRunLen;
  const int per = ns / kT;  // 8 or 16
  uint32_t key[kSample / kT];
#pragma unroll
  for (int i = 0; i < kSample / kT; ++i) {
    key[i] = 0u;
    if (i < 8 || per > 8) {
      const int j = t + kT * i;
      const int64_t start = (int64_t)(j / kRunLen) * (n - kRunLen) / (runs - 1);
      key[i] = ordered_key(s[start + j % kRunLen]);
    }
  }
  // Rank m of the threshold among the samples: the samples expected above
  // the k-th score of the row (e = k ns / n) times 1.25, plus 3 standard
  // deviations of that count (sqrt e) and 8, so that a threshold above the
  // k-th score (too few candidates) stays below about one in a million.
  const double e = (double)k * ns / (double)n;
  uint32_t m = (uint32_t)(1.25 * e + 3.0 * __builtin_sqrt(e)) + 8u;
  if (m > (uint32_t)ns) m = ns;
  // Two 11-bit radix steps on the keys: T is the lower edge of the 22-bit
  // prefix bin that holds the m-th largest sample.
  uint32_t prefix = 0;
  uint32_t* hist = L.u.hist;
  for (int step = 0; step < 2; ++step) {
    const int shift = step == 0 ? 21 : 10;
    for (int i = t; i < kHistBins; i += kT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSample / kT; ++i)
      if ((i < 8 || per > 8) && (step == 0 || (key[i] >> 21) == prefix))
        atomicAdd(&hist[(key[i] >> shift) & (kHistBins - 1)], 1u);
    __syncthreads();
    uint32_t c[kHistBins / kT];
    load_bins<kT>(hist, c);
    const Thresh th = block_threshold<kT>(c, m, L.scan);
    m -= th.above;
    prefix = step == 0 ? (uint32_t)th.digit : (prefix << 11) | (uint32_t)th.digit;
  }
  return prefix << 10;
}

template <bool VEC>
__global__ __launch_bounds__(kT) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                        int32_t* __restrict__ row_len, const int32_t* ctx_len,
                                                        int R, int slice, int k, TopkWs w) {
  __shared__ FilterLds L;
  const int t = threadIdx.x;
  const int row = blockIdx.y;
  const int64_t n = visible_len(row_len, ctx_len, R, row);
  if (ctx_len && blockIdx.x == 0 && t == 0) row_len[row] = (int32_t)n;  // published for the caller
  if (n <= k) return;  // the final kernel emits every position
  const float* s = scores + (size_t)row * ld;
  const uint32_t T = sample_threshold(s, n, k, L);
  const int64_t s0 = (int64_t)blockIdx.x * slice;
  const int64_t s1 = s0 + slice < n ? s0 + slice : n;
  const uint32_t sub = (uint32_t)(w.cap / gridDim.x);  // this slice's share of the row's buffer
  uint2* gcand = w.cand + (size_t)row * w.cap + (size_t)blockIdx.x * sub;
  if (t == 0) L.cnt = 0;
  __syncthreads();

  // Each lane classifies 16 scores per step into a bitmask; one LDS atomic
  // per wave reserves the slots (uniform trip counts). The next step's
  // scores are loaded before the current ones are classified.
  const int lane = t & 63, wave = t >> 6;
  auto load_step = [&](int64_t base, float (&v)[16]) {
    const int64_t wbase = base + 1024 * wave + 4 * lane;  // element (q, e): wbase + 256 q + e
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
  };
  float cur[16], nxt[16];
  if (s0 < s1) load_step(s0, cur);
  for (int64_t base = s0; base < s1; base += 16 * kT) {
    const bool more = base + 16 * kT < s1;
    if (more) load_step(base + 16 * kT, nxt);
    const int64_t wbase = base + 1024 * wave + 4 * lane;
    uint32_t cmask = 0;
    uint32_t keys[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t i = wbase + 256 * (j >> 2) + (j & 3);
      keys[j] = ordered_key(cur[j]);
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
      if (slot < (uint32_t)kListLds) L.u.list[slot] = e;  // the rest of the region takes the overflow
      else if (slot < sub) gcand[slot] = e;
      ++slot;
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < 16; ++j) cur[j] = nxt[j];
    }
  }
  __syncthreads();
  // The true count is published even when it overflowed the slice's region:
  // the final kernel then falls back to the whole row.
  const uint32_t nc = L.cnt;
  const uint32_t keep = nc <= sub ? (nc < (uint32_t)kListLds ? nc : (uint32_t)kListLds) : 0u;
  for (uint32_t i = t; i < keep; i += kT) gcand[i] = L.u.list[i];
  if (t == 0) w.cnt[(size_t)row * kMaxSlices + blockIdx.x] = nc;
}

// ------------------------------------------------------------------ final

static constexpr int kBinLds = 2048;  // threshold-bin elements kept for the last steps

struct FinalLds {
  ScanLds<kTF> scan;
  MinMaxLds<kTF> mm;
  uint32_t emitted;
  uint32_t nbin;
  uint32_t off[kMaxSlices];
  uint32_t total;
  uint32_t bad;
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
  for (int64_t i = t; i < count; i += kTF) {
    const uint64_t c = comp_at(i);
    lo = c < lo ? c : lo;
    hi = c > hi ? c : hi;
  }
  block_minmax<kTF>(lo, hi, L.mm);
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
  for (int i = t; i < kHistBins; i += kTF) L.hist[i] = 0;
  __syncthreads();
  for (int64_t i = t; i < count; i += kTF)
    atomicAdd(&L.hist[(comp_at(i) >> lo_bit) & ((1ull << width) - 1)], 1u);
  __syncthreads();
  uint32_t cnt[kHistBins / kTF];
  load_bins<kTF>(L.hist, cnt);
  Thresh th = block_threshold<kTF>(cnt, need, L.scan);
  const uint64_t b = (shift == 64 ? 0 : prefix << width) | (uint64_t)th.digit;  // top (64 - b_shift) bits
  const int b_shift = lo_bit;
  const bool gather = th.at <= (uint32_t)kBinLds;
  // emit everything above b; gather b
  for (int64_t base = 0; base < count; base += kTF) {
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
      for (uint32_t i = t; i < th.at; i += kTF) out[emitted0 + i] = (int32_t)~(uint32_t)L.bin[i];
    } else {
      if (t == 0) L.emitted = 0;
      __syncthreads();
      for (int64_t base = 0; base < count; base += kTF) {
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
    for (int i = t; i < kHistBins; i += kTF) L.hist[i] = 0;
    __syncthreads();
    for (int64_t j = t; j < nb; j += kTF) {
      const uint64_t c = bin_at(j);
      if ((c >> shift) == prefix) atomicAdd(&L.hist[(c >> lo_bit) & ((1ull << width) - 1)], 1u);
    }
    __syncthreads();
    load_bins<kTF>(L.hist, cnt);
    th = block_threshold<kTF>(cnt, need, L.scan);
    need -= th.above;
    prefix = (prefix << width) | (uint64_t)th.digit;
    shift = lo_bit;
    if (th.at == need || shift == 0) break;
  }
  if (t == 0) L.emitted = 0;
  __syncthreads();
  // elements of b whose top (64 - shift) bits are at least the resolved prefix
  for (int64_t base = 0; base < nb; base += kTF) {
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
__global__ __launch_bounds__(kTF) void topk_final_kernel(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ row_len, const int32_t* ctx_len,
                                                       int R, int slices, int k, int32_t* __restrict__ idx,
                                                       TopkWs w) {
  __shared__ FinalLds L;
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const int64_t n = visible_len(row_len, ctx_len, R, row);
  int32_t* out = idx + (size_t)row * k;
  if (n <= k) {  // every visible position is selected; the rest is padding
    for (int64_t i = t; i < k; i += kTF) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  // slices' counts and their offsets in LDS: lane t of wave 0 owns slice t
  const uint32_t sub = (uint32_t)(w.cap / slices);
  if (t < 64) {
    const uint32_t c = t < slices ? w.cnt[(size_t)row * kMaxSlices + t] : 0u;
    const uint64_t bad = __ballot(c > sub);
    uint32_t incl = c;  // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t x = __shfl_up(incl, d);
      if (t >= d) incl += x;
    }
    L.off[t] = incl - c;
    if (t == 63) L.total = incl;
    if (t == 0) L.bad = bad != 0;
  }
  __syncthreads();
  const uint32_t count = L.total;
  if (!L.bad && count >= (uint32_t)k && count <= (uint32_t)kFinalLds) {
    // element i sits in the last slice whose offset is <= i; eight loads in
    // flight per lane
    const uint2* base = w.cand + (size_t)row * w.cap;
    for (uint32_t b0 = 0; b0 < count; b0 += 8 * kTF) {
      uint2 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t i = b0 + t + j * kTF;
        v[j] = make_uint2(0u, 0u);
        if (i < count) {
          int sl = 0;
#pragma unroll
          for (int step = kMaxSlices / 2; step >= 1; step >>= 1)
            if (sl + step < slices && L.off[sl + step] <= i) sl += step;
          v[j] = base[(size_t)sl * sub + (i - L.off[sl])];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t i = b0 + t + j * kTF;
        if (i < count) L.elems[i] = v[j];
      }
    }
    __syncthreads();
    select_top(L, count, k, out, [&](int64_t i) { return composite(L.elems[i].x, L.elems[i].y); });
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
  // Filter: enough workgroups to cover the GPU twice, at least 4096 scores
  // and at most kMaxSlices workgroups per row.
  int64_t want = (512 + rows - 1) / rows;
  const int64_t max_slices = (max_len + 4095) / 4096;
  if (want > max_slices) want = max_slices;
  if (want > kMaxSlices) want = kMaxSlices;
  if (want < 1) want = 1;
  int64_t slice = (max_len + want - 1) / want;
  slice = (slice + 4095) / 4096 * 4096;
  const int ns = (int)((max_len + slice - 1) / slice);
  if (vec_ok(scores, ld))
    hipLaunchKernelGGL(topk_filter_kernel<true>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len, ctx_len, R,
                       (int)slice, k, w);
  else
    hipLaunchKernelGGL(topk_filter_kernel<false>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len, ctx_len,
                       R, (int)slice, k, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_final_kernel, dim3(rows), dim3(kTF), 0, st, scores, ld, row_len, ctx_len, R, ns, k, idx,
                     w);
  return hipGetLastError();
}

}  // namespace dsa
