// Wave and workgroup primitives of the exact top-k selection, and the
// sampled threshold that every selection path starts from (shared by the
// top-k kernels and by the decode scorer's sampling pass).
#pragma once

#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int kSample = 4096;     // most scores sampled per row
static constexpr int kRunLen = 128;      // ... in evenly spaced runs of this length
static constexpr int kTakeAll = 8192;    // rows up to this length keep every element

// ------------------------------------------------------------------ helpers

// Cross-lane moves through DPP (a VALU operand modifier, a few cycles) rather
// than ds_bpermute (an LDS round trip of ~300 cycles): lanes whose source is
// outside the pattern, or whose row is masked off, read 0.
template <int CTRL, int ROW_MASK = 0xf>
DSA_DEV uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, true);
}
constexpr int kDppXor1 = 0xb1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane 7 - i within each 8
constexpr int kDppMirror = 0x140;      // lane 15 - i within each 16
constexpr int kDppShr1 = 0x111;        // row_shr:n = 0x110 + n
constexpr int kDppBcast15 = 0x142;     // lane 15 of each row -> the next row
constexpr int kDppBcast31 = 0x143;     // lane 31 -> rows 2 and 3

// Inclusive prefix sum over the 64 lanes (Hillis-Steele inside rows of 16,
// then the row totals carried across with the row broadcasts).
DSA_DEV uint32_t wave_incl_sum(uint32_t x) {
  x += dpp<kDppShr1>(x);
  x += dpp<kDppShr1 + 1>(x);
  x += dpp<kDppShr1 + 3>(x);
  x += dpp<kDppShr1 + 7>(x);
  x += dpp<kDppBcast15, 0xa>(x);
  x += dpp<kDppBcast31, 0xc>(x);
  return x;
}

// 64-bit value of lane ^ 1, ^ 2 or the mirrored lane, one DPP move per half.
template <int CTRL>
DSA_DEV uint64_t dpp64(uint64_t v) {
  return ((uint64_t)dpp<CTRL>((uint32_t)(v >> 32)) << 32) | dpp<CTRL>((uint32_t)v);
}

// Max over the wave, returned in every lane (uniform).
DSA_DEV uint32_t wave_max32(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  return max(max((uint32_t)__builtin_amdgcn_readlane(v, 0), (uint32_t)__builtin_amdgcn_readlane(v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane(v, 32), (uint32_t)__builtin_amdgcn_readlane(v, 48)));
}

// Min and max over the wave, returned in every lane (uniform).
DSA_DEV void wave_minmax64(uint64_t& lo, uint64_t& hi) {
#define DSA_MINMAX_STEP(CTRL)                       \
  {                                                 \
    const uint64_t a = dpp64<CTRL>(lo), b = dpp64<CTRL>(hi); \
    lo = a < lo ? a : lo;                           \
    hi = b > hi ? b : hi;                           \
  }
  DSA_MINMAX_STEP(kDppXor1)
  DSA_MINMAX_STEP(kDppXor2)
  DSA_MINMAX_STEP(kDppHalfMirror)
  DSA_MINMAX_STEP(kDppMirror)
#undef DSA_MINMAX_STEP
  // every lane of a row now holds the row's result; combine the four rows
  uint64_t l = ~0ull, h = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t a = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(lo >> 32), 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((uint32_t)lo, 16 * r);
    const uint64_t b = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(hi >> 32), 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((uint32_t)hi, 16 * r);
    l = a < l ? a : l;
    h = b > h ? b : h;
  }
  lo = l;
  hi = h;
}

// Append the predicated lanes of a wave to a counter (LDS or global); returns
// each predicated lane's slot. One atomic per wave.
DSA_DEV uint32_t wave_append(uint32_t* counter, bool pred) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return 0;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
  base = __builtin_amdgcn_readlane(base, leader);
  const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  return base + below;
}

// Exclusive prefix of small per-lane counts (below 2^BITS) over the wave,
// from BITS bit-sliced ballots (no LDS traffic); total is the wave sum.
template <int BITS = 5>
DSA_DEV uint32_t wave_prefix_small(uint32_t cnt, uint32_t& total) {
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int bit = 0; bit < BITS; ++bit) {
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
  const uint32_t pre = wave_incl_sum(mine);
  const uint32_t wtot = __builtin_amdgcn_readlane(pre, 63);
  if (lane == 0) s.wsum[wave] = wtot;
  if (t == 0) s.res[0] = s.res[1] = s.res[2] = 0;
  __syncthreads();
  // bins of the later lanes of this wave, plus the later waves' totals (lane
  // w < NT / 64 reads wave w's total: one LDS read per lane)
  const uint32_t later = (lane < NT / 64 && lane > wave) ? s.wsum[lane] : 0u;
  uint32_t above = wtot - pre + __builtin_amdgcn_readlane(wave_incl_sum(later), 63);
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
  // No barrier after this read: every caller passes at least two more
  // barriers before the next call clears res.
  return Thresh{(int)s.res[0], s.res[1], s.res[2]};
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
  wave_minmax64(lo, hi);
  if (lane == 0) {
    s.lo[wave] = lo;
    s.hi[wave] = hi;
  }
  __syncthreads();
  // lane w < NT / 64 takes wave w's result; one more wave reduction
  lo = lane < NT / 64 ? s.lo[lane] : ~0ull;
  hi = lane < NT / 64 ? s.hi[lane] : 0ull;
  wave_minmax64(lo, hi);
  __syncthreads();
}

// ------------------------------------------------------------------ filter

// Visible length of a row: from row_len, or derived in the fused decode.
// Clamped to [0, ld], so that a length beyond the row's storage never turns
// into an out-of-bounds read.
DSA_DEV int64_t visible_len(const int32_t* row_len, const int32_t* ctx_len, int R, int row, int64_t ld) {
  const int64_t n = ctx_len ? (int64_t)ctx_len[row / R] - R + row % R + 1 : (int64_t)row_len[row];
  return n < 0 ? 0 : (n > ld ? ld : n);
}

// Sampled threshold of a row (the same in every workgroup of it), in two
// parts so that a caller can issue other loads in between.
// sample_load: ns samples (2048, or 4096 past 256K elements); sample j
// (thread t of NT takes j = t + NT i) is element (j % 128) of run j / 128, the
// runs evenly spaced over the row.
template <int NT>
DSA_DEV void sample_load(const float* __restrict__ s, int64_t n, uint32_t (&raw)[kSample / NT]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kSample / NT; ++i) raw[i] = 0u;
  if (n <= kTakeAll) return;  // no samples needed (uniform)
  const int ns = n > (1 << 18) ? 4096 : 2048;
  const int per = ns / NT;
  // Run r starts at floor(r span / d), span = n - 128, d = runs - 1 (31 or
  // 15) = r q + floor(r rem / d) with q, rem = span divided by d, computed
  // once; r rem < d^2 takes a constant-divisor 32-bit division (a 64-bit
  // division by a variable would be a long software routine per sample).
  // Every load is issued before any is used: the raw bits are converted to
  // keys where they are first needed.
  const uint32_t span = (uint32_t)(n - kRunLen);  // rows are shorter than 2^31
  const bool wide = ns == 4096;
  const uint32_t q = wide ? span / 31u : span / 15u;
  const uint32_t rem = span - q * (wide ? 31u : 15u);
#pragma unroll
  for (int i = 0; i < kSample / NT; ++i) {
    const uint32_t j = (uint32_t)(t + NT * i);
    const uint32_t r = j / kRunLen;
    const uint32_t start = r * q + (wide ? (r * rem) / 31u : (r * rem) / 15u);
    const size_t pos = i < per ? (size_t)start + j % kRunLen : 0;  // extra slots re-read position 0
    raw[i] = __float_as_uint(s[pos]);
  }
}

// sample_select: the ordered-key threshold T from the samples; every element
// is kept (T = 0) for rows of at most kTakeAll elements. Thread t holds
// samples t + NT i (i < NS / NT; NS bounds the sample count).
template <int NT, int NS = kSample>
DSA_DEV uint32_t sample_select(const uint32_t (&raw)[NS / NT], int64_t n, int k, uint32_t* hist,
                               ScanLds<NT>& scan, int ns_given = 0) {
  const int t = threadIdx.x;
  if (n <= kTakeAll) return 0u;
  // ns_given: the number of samples when the caller drew its own
  const int ns = ns_given > 0 ? ns_given : (n > (1 << 18) ? 4096 : 2048);
  const int per = ns / NT;
  uint32_t key[NS / NT];
#pragma unroll
  for (int i = 0; i < NS / NT; ++i) key[i] = ordered_key(__uint_as_float(raw[i]));
  // Rank m of the threshold among the samples: the samples expected above
  // the k-th score of the row (e = k ns / n) times 1.25, plus 3 standard
  // deviations of that count (sqrt e) and 8, so that a threshold above the
  // k-th score (too few candidates) stays below about one in a million.
  const double e = (double)k * ns / (double)n;
  uint32_t m = (uint32_t)(1.25 * e + 3.0 * __builtin_sqrt(e)) + 8u;
  if (m > (uint32_t)ns) m = ns;
  // 11-bit radix steps that start just below the prefix every sample shares
  // (from their min and max, so that the first step spreads over its bins):
  // T is the lower edge of the bin that holds the m-th largest sample, once
  // the bin is at most 2^10 keys wide.
  const int lane = t & 63, wave = t >> 6;
  uint32_t lo = ~0u, hi = 0u;
#pragma unroll
  for (int i = 0; i < NS / NT; ++i)
    if (i < per) {
      lo = min(lo, key[i]);
      hi = max(hi, key[i]);
    }
  lo = ~wave_max32(~lo);
  hi = wave_max32(hi);
  if (lane == 0) {
    hist[wave] = lo;
    hist[NT / 64 + wave] = hi;
  }
  __syncthreads();
  lo = ~wave_max32(lane < NT / 64 ? ~hist[lane] : 0u);
  hi = wave_max32(lane < NT / 64 ? hist[NT / 64 + lane] : 0u);
  __syncthreads();  // the extremes are read before the histogram is cleared
  if (lo == hi) return hi;  // every sample has the same key (uniform branch)
  int shift = 32 - __clz((int)(lo ^ hi));  // bits below the shared prefix
  uint32_t prefix = shift == 32 ? 0u : hi >> shift;
  while (true) {  // uniform trip count
    const int width = shift < 11 ? shift : 11;
    const int lo_bit = shift - width;
    for (int i = t; i < kHistBins; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NS / NT; ++i)
      if (i < per && (shift == 32 || (key[i] >> shift) == prefix))
        atomicAdd(&hist[(key[i] >> lo_bit) & ((1u << width) - 1)], 1u);
    __syncthreads();
    uint32_t c[kHistBins / NT];
    load_bins<NT>(hist, c);
    const Thresh th = block_threshold<NT>(c, m, scan);
    m -= th.above;
    prefix = (shift == 32 ? 0u : prefix << width) | (uint32_t)th.digit;
    shift = lo_bit;
    if (shift <= 10) return prefix << shift;
    // (every thread read its bins before block_threshold's first barrier, so
    // the next clear is safe)
  }
}

// key >= T as a float comparison (scores are not NaN): T is the lower edge of
// a bin holding a sampled score, so its float is a number unless T lies below
// every number's key, where every score passes.
DSA_DEV float key_threshold_float(uint32_t T) {
  return T <= ordered_key(-INFINITY) ? -INFINITY : __uint_as_float((T & 0x80000000u) ? (T & 0x7fffffffu) : ~T);
}

// ------------------------------------------------------------------ exact selection

static constexpr int kTF = 1024;  // threads of a selecting workgroup

static constexpr int kBinLds = 2048;  // threshold-bin elements kept for the last steps

// LDS of select_top (one workgroup of kTF threads).
struct SelectLds {
  ScanLds<kTF> scan;
  MinMaxLds<kTF> mm;
  uint32_t emitted;
  uint32_t nbin;
  uint32_t hist[kHistBins];
  uint64_t bin[kBinLds];
};


// Emit the positions of the k largest composites among `count` elements
// (comp_at(i) gives element i's composite).
//  1. The radix digits start below the bits every element shares (the
//     survivors of one row have close scores: their top bits would all fall
//     in one bin).
//  2. One 11-bit step finds the bin b holding the k-th largest; a second
//     pass emits everything above b and gathers b's elements into LDS.
//  3. Further 11-bit steps over the gathered elements resolve the rest
//     (without the gather, when b holds more than kBinLds elements); a bin
//     of at most 64 elements is ranked by one wave instead.
// Where the i-th selected position goes: out[i], and with a page table also
// its physical cache slot (page id * 64 + offset) to slots[i].
struct Emit {
  int32_t* out;
  int32_t* slots;      // or null
  const int32_t* tbl;  // page ids of the row's request (LDS), when slots is set
  DSA_DEV void operator()(uint32_t i, uint32_t pos) const {
    out[i] = (int32_t)pos;
    if (slots) slots[i] = tbl[pos >> 6] * kBlock + (int32_t)(pos & 63);
  }
};

// With have_bounds, [lo0, hi0] is given to hold every composite (the pass
// that finds the exact extremes is skipped).
template <class CompAt>
DSA_DEV void select_top(SelectLds& L, int64_t count, int k, const Emit& out, CompAt comp_at,
                        bool have_bounds = false, uint64_t lo0 = 0, uint64_t hi0 = 0) {
  const int t = threadIdx.x;
  uint64_t lo = lo0, hi = hi0;
  if (!have_bounds) {
    lo = ~0ull;
    hi = 0;
    for (int64_t i = t; i < count; i += kTF) {
      const uint64_t c = comp_at(i);
      lo = c < lo ? c : lo;
      hi = c > hi ? c : hi;
    }
    block_minmax<kTF>(lo, hi, L.mm);
  }
  if (t == 0) {
    L.emitted = 0;
    L.nbin = 0;
  }
  // the composites are distinct, so lo == hi only for a single element
  if (lo == hi) {
    if (t == 0) out(0, ~(uint32_t)hi);
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
  // emit everything above b; gather b. Each thread counts its elements of
  // both kinds first, so that a wave reserves its slots with one atomic per
  // kind instead of one per pass over 1024 elements.
  {
    uint32_t na = 0, nb = 0;
    for (int64_t i = t; i < count; i += kTF) {
      const uint64_t c = comp_at(i);
      na += (uint32_t)((c >> b_shift) > b);
      nb += (uint32_t)(gather && (c >> b_shift) == b);
    }
    const uint32_t ia = wave_incl_sum(na), ib = wave_incl_sum(nb);
    uint32_t sa = wave_reserve(&L.emitted, __builtin_amdgcn_readlane(ia, 63)) + ia - na;
    uint32_t sb = wave_reserve(&L.nbin, __builtin_amdgcn_readlane(ib, 63)) + ib - nb;
    for (int64_t i = t; i < count; i += kTF) {
      const uint64_t c = comp_at(i);
      if ((c >> b_shift) > b) {
        if (sa < (uint32_t)k) out(sa, ~(uint32_t)c);
        ++sa;
      } else if (gather && (c >> b_shift) == b) {
        if (sb < (uint32_t)kBinLds) L.bin[sb] = c;
        ++sb;
      }
    }
  }
  __syncthreads();
  need -= th.above;
  const uint32_t emitted0 = th.above;
  if (th.at == need) {  // all of b is selected
    if (gather) {
      for (uint32_t i = t; i < th.at && emitted0 + i < (uint32_t)k; i += kTF)
        out(emitted0 + i, ~(uint32_t)L.bin[i]);
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
        if (take && emitted0 + slot < (uint32_t)k) out(emitted0 + slot, ~(uint32_t)c);
      }
    }
    return;
  }
  // a bin of at most 64 gathered elements: the first wave ranks them (each
  // lane counts the larger composites of the bin; they are distinct) and
  // emits the `need` largest, with no more barriers
  if (gather && th.at <= 64) {
    if (t < 64) {
      const uint32_t nbin = th.at;
      const uint64_t c = (uint32_t)t < nbin ? L.bin[t] : 0ull;
      uint32_t rank = 0;
      for (uint32_t j = 0; j < nbin; ++j) {  // uniform trip count
        const uint64_t cj = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(c >> 32), j) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((uint32_t)c, j);
        rank += cj > c ? 1u : 0u;
      }
      if ((uint32_t)t < nbin && rank < need) out(emitted0 + rank, ~(uint32_t)c);
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
    if (take && emitted0 + slot < (uint32_t)k) out(emitted0 + slot, ~(uint32_t)c);
  }
}

// Rows of at most k visible positions: all of them, then -1 padding (and
// their physical slots when asked for).
DSA_DEV void emit_all_positions(int row, int R, int64_t n, int k, int32_t* out, const SlotOut& so) {
  const int t = threadIdx.x;
  for (int64_t i = t; i < k; i += kTF) out[i] = i < n ? (int32_t)i : -1;
  if (so.slots) {
    const int32_t* table = so.block_table + (size_t)(row / R) * so.max_blocks;
    for (int i = t; i < k; i += kTF)
      so.slots[(size_t)row * k + i] = i < n && (i >> 6) < so.max_blocks ? table[i >> 6] * kBlock + (i & 63) : -1;
  }
}

// Physical slots of a row's written selection (rows this long have too many
// pages to stage their table in LDS): every thread translates its entries
// with all its loads in flight. The caller makes `out` workgroup-visible.
DSA_DEV void emit_slots(int row, int R, int k, const int32_t* out, const SlotOut& so) {
  const int t = threadIdx.x;
  const int32_t* table = so.block_table + (size_t)(row / R) * so.max_blocks;
  constexpr int kPer = (kMaxTopk + kTF - 1) / kTF;
  int32_t pos[kPer], page[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = t + j * kTF;
    pos[j] = i < k ? out[i] : -1;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) page[j] = pos[j] >= 0 && (pos[j] >> 6) < so.max_blocks ? table[pos[j] >> 6] : -1;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = t + j * kTF;
    if (i < k) so.slots[(size_t)row * k + i] = page[j] >= 0 ? page[j] * kBlock + (pos[j] & 63) : -1;
  }
}

// ------------------------------------------------------------------ scorer work split

// The decode scorer hands its G workgroups (per row group) to the B
// requests in proportion to their pages: request b owns workgroups
// [W(b), W(b + 1)) with W(b) = b + floor((G - B) * S_b / P), where S_b
// counts the pages of the requests before b and P those of all requests.
// Every request gets at least one workgroup (G >= B) and each workgroup
// about P / (G - B) pages, whatever the mix of lengths ("vLLM Day-0 Support
// for Kimi K3.1 Pro", section "Fused low-latency decode for DSA layers": a
// key-balanced scorer; "TokenSpeed Kimi K3.1", section "Reducing indexer
// overhead on AMD MI350X": kernels size their work from each request's
// actual length). Computed from ctx_len alone, by one wave (every lane
// takes part; the result is uniform), so the candidate selection can
// recompute exactly the split the scorer used. The floors are taken in
// double precision: (G - B) * S_b is an integer below 2^53, so both sides
// get the same values and W(B) = G.
struct WgRange {
  int b;      // request
  int first;  // W(b)
  int count;  // W(b + 1) - W(b)
};

DSA_DEV int pages_of(const int32_t* ctx_len, int b) {
  const int L = ctx_len[b];
  return L > 0 ? (L + kBlock - 1) / kBlock : 0;
}

// want_b < 0: the request owning workgroup x (0 <= x < G); else request want_b.
DSA_DEV WgRange wg_range(const int32_t* ctx_len, int B, int G, int x, int want_b) {
  const int lane = threadIdx.x & 63;
  double P = 0.0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const uint32_t pg = b < B ? (uint32_t)pages_of(ctx_len, b) : 0u;
    P += (double)__builtin_amdgcn_readlane(wave_incl_sum(pg), 63);
  }
  const double spare = (double)(G - B);
  double S = 0.0;
  WgRange r{0, 0, 1};
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const uint32_t pg = b < B ? (uint32_t)pages_of(ctx_len, b) : 0u;
    const uint32_t incl = wave_incl_sum(pg);
    const double P_safe = P > 0.0 ? P : 1.0;
    const int w0 = b + (int)__builtin_floor(spare * (S + (double)(incl - pg)) / P_safe);
    const int w1 = b + 1 + (int)__builtin_floor(spare * (S + (double)incl) / P_safe);
    const bool mine = b < B && (want_b < 0 ? (w0 <= x && x < w1) : b == want_b);
    const uint64_t m = __ballot(mine);
    if (m) {
      const int l = __ffsll((unsigned long long)m) - 1;
      r.b = __builtin_amdgcn_readlane(b, l);
      r.first = __builtin_amdgcn_readlane(w0, l);
      r.count = __builtin_amdgcn_readlane(w1, l) - r.first;
      return r;
    }
    S += (double)__builtin_amdgcn_readlane(incl, 63);
  }
  return r;
}

}  // namespace dsa
