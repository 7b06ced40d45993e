// Exact top-k selection by radix select over ordered fp32 keys.
//
// "TokenSpeed Kimi K3.1", step 3: a radix top-k keeps the 2,048
// highest-scoring positions per query row; section "Reducing indexer overhead
// on AMD MI350X": one row is spread over several workgroups that share a
// histogram of score prefixes, because one workgroup per row would leave most
// of the 256 compute units idle at 4-16 decode rows.
//
// Every element is ranked by the 64-bit composite (ordered score key << 32) |
// ~position, which is unique: larger score first, then lower position. The
// top k composites are therefore a unique set, the same on every run.
//
// Kernels, all on one stream:
//  clear   zero each row's 2048-bin histogram and counters (a fill kernel, so
//          the sequence stays safe under stream capture);
//  hist    first digit (top 11 key bits) histogram, several workgroups per
//          row; the decode scorer can build it instead;
//  select  every workgroup reads the row histogram, finds the threshold bin
//          b1, streams its slice of the row with 16-byte loads and compacts
//          the positions above b1 and the (key, position) candidates inside
//          b1 into LDS lists, which it appends to the output and to a global
//          candidate buffer with one atomic per list; it also counts the
//          candidates' second digit (next 11 bits) into a row histogram;
//  refine  one workgroup per row finds the second-digit threshold b2, emits
//          the candidates above it in one pass over the list, and resolves
//          the few b2 candidates (remaining key bits, then positions) in LDS.
#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int kT = 256;             // threads per workgroup
static constexpr int kWinLds = 2048;       // winners one workgroup can hold (bounded by k)
static constexpr int kCandLds = 2048;      // candidates kept in LDS before spilling to global
static constexpr int kRefineLds = 4096;    // candidates the refine resolves in LDS

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Candidate slots per row: the whole row when a 64 MB buffer allows it,
// else 64 MB spread over the rows, never fewer than 8192.
static int32_t cand_cap(int rows, int64_t max_len) {
  int64_t c = (int64_t)(64ll << 20) / 8 / (rows > 0 ? rows : 1);
  if (c > max_len) c = max_len;
  if (c < 8192) c = 8192;
  return (int32_t)((c + 63) / 64 * 64);
}

// hist holds two 2048-bin histograms per row: the first digit (top 11 key
// bits) of every score and the second digit (next 11 bits) of the candidates.
size_t topk_ws_bytes(int rows, int64_t max_len) {
  const size_t hist = align_up((size_t)rows * 2 * kHistBins * 4, 256);
  const size_t ctr = align_up((size_t)rows * 4 * 4, 256);
  const size_t cand = align_up((size_t)rows * cand_cap(rows, max_len) * 8, 256);
  return hist + ctr + cand;
}

TopkWs topk_ws_carve(void* ws, int rows, int64_t max_len) {
  TopkWs w;
  char* p = static_cast<char*>(ws);
  w.hist = reinterpret_cast<uint32_t*>(p);
  w.hist2 = w.hist + (size_t)rows * kHistBins;
  p += align_up((size_t)rows * 2 * kHistBins * 4, 256);
  w.ctr = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * 4 * 4, 256);
  w.cand = reinterpret_cast<uint2*>(p);
  w.cap = cand_cap(rows, max_len);
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

DSA_DEV uint64_t composite(uint32_t key, uint32_t pos) { return ((uint64_t)key << 32) | (uint64_t)(~pos); }

// ------------------------------------------------------------------ kernels

__global__ void topk_clear_kernel(uint32_t* hist, uint32_t* ctr, int rows, int32_t* row_len,
                                  const int32_t* ctx_len, int R) {
  const size_t nh = (size_t)rows * 2 * kHistBins / 4;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4* h4 = reinterpret_cast<u32x4*>(hist);
  for (size_t j = i; j < nh; j += stride) h4[j] = u32x4{0u, 0u, 0u, 0u};
  for (size_t j = i; j < (size_t)rows * 4; j += stride) ctr[j] = 0;
  if (row_len)
    for (size_t j = i; j < (size_t)rows; j += stride) row_len[j] = ctx_len[j / R] - R + (int)(j % R) + 1;
}

template <bool VEC>
__global__ __launch_bounds__(kT) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                      const int32_t* __restrict__ row_len, int slice,
                                                      uint32_t* __restrict__ hist) {
  __shared__ uint32_t lh[kHistBins];
  const int row = blockIdx.y;
  for (int i = threadIdx.x; i < kHistBins; i += kT) lh[i] = 0;
  __syncthreads();
  const int64_t n = row_len[row];
  const int64_t s0 = (int64_t)blockIdx.x * slice;
  const int64_t s1 = s0 + slice < n ? s0 + slice : n;
  const float* s = scores + (size_t)row * ld;
  if (VEC) {
    for (int64_t i = s0 + 4 * threadIdx.x; i < s1; i += 4 * kT) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(s + i);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < s1) atomicAdd(&lh[ordered_key(v[e]) >> 21], 1u);
    }
  } else {
    for (int64_t i = s0 + threadIdx.x; i < s1; i += kT) atomicAdd(&lh[ordered_key(s[i]) >> 21], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += kT)
    if (lh[i]) atomicAdd(&hist[(size_t)row * kHistBins + i], lh[i]);
}

struct SelectLds {
  ScanLds scan;
  uint32_t cnt[2];   // LDS list lengths: winners, candidates
  uint32_t base[2];  // global slots reserved for them
  uint32_t emitted;
  union {
    struct {
      uint32_t win[kWinLds];
      uint2 cand[kCandLds];
      uint32_t hist2[kHistBins];
    } sel;
    struct {
      uint32_t hist[kHistBins];
      uint2 elems[kRefineLds];
    } ref;
  } u;
};

// Resolve the rest of one row's selection among its first-digit candidates.
// Runs in one workgroup; `above` positions are already in the output.
DSA_DEV void refine_row(SelectLds& L, const float* __restrict__ s, int64_t n, uint64_t b1, uint32_t above,
                        uint32_t at, int k, int32_t* __restrict__ out, const uint2* __restrict__ gcand, int cap) {
  const int t = threadIdx.x;
  // Source of the candidates: LDS copy, the global buffer, or (overflow) the whole row.
  const int src = at <= (uint32_t)kRefineLds ? 0 : (at <= (uint32_t)cap ? 1 : 2);
  const int64_t count = src == 2 ? n : (int64_t)at;
  if (src == 0)
    for (int64_t i = t; i < count; i += kT) L.u.ref.elems[i] = gcand[i];
  if (t == 0) L.emitted = 0;
  __syncthreads();
  auto comp_at = [&](int64_t i) -> uint64_t {
    if (src == 0) return composite(L.u.ref.elems[i].x, L.u.ref.elems[i].y);
    if (src == 1) return composite(gcand[i].x, gcand[i].y);
    return composite(ordered_key(s[i]), (uint32_t)i);
  };
  uint32_t need = (uint32_t)k - above;
  uint64_t prefix = b1;
  int shift = 53;
  while (true) {
    const int width = shift < 11 ? shift : 11;
    const int lo = shift - width;
    const uint64_t mask = (1ull << width) - 1;
    for (int i = t; i < kHistBins; i += kT) L.u.ref.hist[i] = 0;
    __syncthreads();
    for (int64_t i = t; i < count; i += kT) {
      const uint64_t c = comp_at(i);
      if ((c >> shift) == prefix) atomicAdd(&L.u.ref.hist[(c >> lo) & mask], 1u);
    }
    __syncthreads();
    uint32_t cnt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt[i] = L.u.ref.hist[8 * t + i];
    const Thresh th = block_threshold(cnt, need, L.scan);
    need -= th.above;
    prefix = (prefix << width) | (uint64_t)th.digit;
    shift = lo;
    if (th.at == need || shift == 0) break;
  }
  // Everything in bin b1 whose composite prefix is at least the resolved one.
  for (int64_t base = 0; base < count; base += kT) {
    const int64_t i = base + t;
    bool take = false;
    uint32_t pos = 0;
    if (i < count) {
      const uint64_t c = comp_at(i);
      take = (c >> 53) == b1 && (c >> shift) >= prefix;
      pos = ~(uint32_t)c;
    }
    const uint32_t slot = wave_append(&L.emitted, take);
    if (take && above + slot < (uint32_t)k) out[above + slot] = (int32_t)pos;
  }
}

// The row's candidates (all of bin b1) are in gcand and their second-digit
// histogram in hist2. Find the second digit b2 of the need-th largest, emit
// candidates above it while scanning the list once, gather the b2 ones into
// LDS and resolve them there (or, if they overflow LDS, from the list).
DSA_DEV void refine_from_cands(SelectLds& L, uint64_t b1, uint32_t above, uint32_t at, int k,
                               int32_t* __restrict__ out, const uint2* __restrict__ gcand,
                               const uint32_t* __restrict__ hist2) {
  const int t = threadIdx.x;
  uint32_t c[8];
  {
    const u32x4* h = reinterpret_cast<const u32x4*>(hist2 + 8 * t);
    const u32x4 a = h[0], b = h[1];
    c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
    c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
  }
  if (t == 0) {
    L.emitted = 0;
    L.cnt[1] = 0;
  }
  const uint32_t need = (uint32_t)k - above;
  const Thresh th = block_threshold(c, need, L.scan);
  const uint32_t b2 = (uint32_t)th.digit;
  const bool fits = th.at <= (uint32_t)kRefineLds;
  // 8 candidates per lane per step: one atomic per wave and list.
  for (int64_t base = 0; base < (int64_t)at; base += 8 * kT) {
    uint2 e[8];
    uint32_t hmask = 0, emask = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t i = base + t + (int64_t)kT * j;
      e[j] = make_uint2(0u, 0u);
      if (i < (int64_t)at) {
        e[j] = gcand[i];
        const uint32_t d2 = (e[j].x >> 10) & (kHistBins - 1);
        hmask |= (uint32_t)(d2 > b2) << j;
        emask |= (uint32_t)(d2 == b2) << j;
      }
    }
    if (!fits) emask = 0;
    uint32_t th_, te;
    const uint32_t ph = wave_prefix_small((uint32_t)__popc(hmask), th_);
    const uint32_t pe = wave_prefix_small((uint32_t)__popc(emask), te);
    const uint32_t bh = wave_reserve(&L.emitted, th_);
    const uint32_t be = wave_reserve(&L.cnt[1], te);
    uint32_t slot = bh + ph;
    while (hmask) {
      const int j = __builtin_ctz(hmask);
      hmask &= hmask - 1;
      if (above + slot < (uint32_t)k) out[above + slot] = (int32_t)e[j].y;
      ++slot;
    }
    slot = be + pe;
    while (emask) {
      const int j = __builtin_ctz(emask);
      emask &= emask - 1;
      if (slot < (uint32_t)kRefineLds) L.u.ref.elems[slot] = e[j];
      ++slot;
    }
  }
  __syncthreads();
  const uint32_t above2 = above + th.above;
  if (th.at == need - th.above) {  // every b2 candidate is selected
    const int64_t cnt = th.at;
    for (int64_t base = 0; base < (fits ? cnt : (int64_t)at); base += kT) {
      const int64_t i = base + t;
      bool take = false;
      uint32_t pos = 0;
      if (fits) {
        if (i < cnt) {
          take = true;
          pos = L.u.ref.elems[i].y;
        }
      } else if (i < (int64_t)at) {
        const uint2 e = gcand[i];
        take = ((e.x >> 10) & (kHistBins - 1)) == b2;
        pos = e.y;
      }
      const uint32_t slot = wave_append(&L.emitted, take);
      if (take && above + slot < (uint32_t)k) out[above + slot] = (int32_t)pos;
    }
    return;
  }
  // Resolve the b2 bin: remaining key bits, then positions.
  const int64_t count = fits ? (int64_t)th.at : (int64_t)at;
  auto comp_at = [&](int64_t i) -> uint64_t {
    const uint2 e = fits ? L.u.ref.elems[i] : gcand[i];
    return composite(e.x, e.y);
  };
  uint32_t need2 = need - th.above;
  uint64_t prefix = (b1 << 11) | b2;
  int shift = 42;
  while (true) {
    const int width = shift < 11 ? shift : 11;
    const int lo = shift - width;
    const uint64_t mask = (1ull << width) - 1;
    for (int i = t; i < kHistBins; i += kT) L.u.ref.hist[i] = 0;
    __syncthreads();
    for (int64_t i = t; i < count; i += kT) {
      const uint64_t cc = comp_at(i);
      if ((cc >> shift) == prefix) atomicAdd(&L.u.ref.hist[(cc >> lo) & mask], 1u);
    }
    __syncthreads();
    uint32_t cnt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt[i] = L.u.ref.hist[8 * t + i];
    const Thresh tr = block_threshold(cnt, need2, L.scan);
    need2 -= tr.above;
    prefix = (prefix << width) | (uint64_t)tr.digit;
    shift = lo;
    if (tr.at == need2 || shift == 0) break;
  }
  for (int64_t base = 0; base < count; base += kT) {
    const int64_t i = base + t;
    bool take = false;
    uint32_t pos = 0;
    if (i < count) {
      const uint64_t cc = comp_at(i);
      take = (cc >> 42) == ((b1 << 11) | b2) && (cc >> shift) >= prefix;
      pos = ~(uint32_t)cc;
    }
    const uint32_t slot = wave_append(&L.emitted, take);
    if (take && above + slot < (uint32_t)k) out[above + slot] = (int32_t)pos;
  }
  (void)above2;
}

template <bool VEC>
__global__ __launch_bounds__(kT) void topk_select_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ row_len, int slice, int k,
                                                        int32_t* __restrict__ idx, TopkWs w) {
  __shared__ SelectLds L;
  const int t = threadIdx.x;
  const int row = blockIdx.y;
  const int64_t n = row_len[row];
  const int64_t s0 = (int64_t)blockIdx.x * slice;
  const int64_t s1 = s0 + slice < n ? s0 + slice : n;
  int32_t* out = idx + (size_t)row * k;
  if (n <= k) {  // every visible position is selected; the rest is padding
    for (int64_t i = s0 + t; i < s1; i += kT) out[i] = (int32_t)i;
    if (blockIdx.x == 0)
      for (int64_t i = n + t; i < k; i += kT) out[i] = -1;
    return;
  }
  uint32_t c[8];
  {
    const u32x4* h = reinterpret_cast<const u32x4*>(w.hist + (size_t)row * kHistBins + 8 * t);
    const u32x4 a = h[0], b = h[1];
    c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
    c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
  }
  if (t == 0) L.cnt[0] = L.cnt[1] = 0;
  for (int i = t; i < kHistBins; i += kT) L.u.sel.hist2[i] = 0;
  const Thresh th = block_threshold(c, (uint32_t)k, L.scan);
  const uint32_t b1 = (uint32_t)th.digit;
  const bool keep = th.at <= (uint32_t)w.cap;
  uint32_t* ctr = w.ctr + (size_t)row * 4;
  uint2* gcand = w.cand + (size_t)row * w.cap;
  const float* s = scores + (size_t)row * ld;

  // Each lane classifies 16 scores per step into win/candidate bitmasks; one
  // LDS atomic per wave and list reserves the slots (uniform trip counts).
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
    uint32_t wmask = 0, cmask = 0;
    uint32_t keys[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t i = wbase + 256 * (j >> 2) + (j & 3);
      keys[j] = ordered_key(v[j]);
      const uint32_t bin = keys[j] >> 21;
      if (i < s1) {
        wmask |= (uint32_t)(bin > b1) << j;
        if (keep && bin == b1) {
          cmask |= 1u << j;
          atomicAdd(&L.u.sel.hist2[(keys[j] >> 10) & (kHistBins - 1)], 1u);
        }
      }
    }
    uint32_t tw, tc;
    const uint32_t pw = wave_prefix_small((uint32_t)__popc(wmask), tw);
    const uint32_t pc = wave_prefix_small((uint32_t)__popc(cmask), tc);
    const uint32_t bw = wave_reserve(&L.cnt[0], tw);
    const uint32_t bc = wave_reserve(&L.cnt[1], tc);
    uint32_t slot = bw + pw;
    while (wmask) {
      const int j = __builtin_ctz(wmask);
      wmask &= wmask - 1;
      if (slot < (uint32_t)kWinLds) L.u.sel.win[slot] = (uint32_t)(wbase + 256 * (j >> 2) + (j & 3));
      ++slot;
    }
    slot = bc + pc;
    while (cmask) {
      const int j = __builtin_ctz(cmask);
      cmask &= cmask - 1;
      const uint2 e = make_uint2(keys[j], (uint32_t)(wbase + 256 * (j >> 2) + (j & 3)));
      if (slot < (uint32_t)kCandLds) {
        L.u.sel.cand[slot] = e;
      } else {
        const uint32_t gs = atomicAdd(&ctr[1], 1u);
        if (gs < (uint32_t)w.cap) gcand[gs] = e;
      }
      ++slot;
    }
  }
  __syncthreads();
  if (t == 0) {
    const uint32_t nw = L.cnt[0] < (uint32_t)kWinLds ? L.cnt[0] : (uint32_t)kWinLds;
    const uint32_t nc = L.cnt[1] < (uint32_t)kCandLds ? L.cnt[1] : (uint32_t)kCandLds;
    L.base[0] = nw ? atomicAdd(&ctr[0], nw) : 0;
    L.base[1] = nc ? atomicAdd(&ctr[1], nc) : 0;
    L.cnt[0] = nw;
    L.cnt[1] = nc;
  }
  __syncthreads();
  for (uint32_t i = t; i < L.cnt[0]; i += kT)
    if (L.base[0] + i < (uint32_t)k) out[L.base[0] + i] = (int32_t)L.u.sel.win[i];
  for (uint32_t i = t; i < L.cnt[1]; i += kT)
    if (L.base[1] + i < (uint32_t)w.cap) gcand[L.base[1] + i] = L.u.sel.cand[i];
  if (keep)
    for (int i = t; i < kHistBins; i += kT)
      if (L.u.sel.hist2[i]) atomicAdd(&w.hist2[(size_t)row * kHistBins + i], L.u.sel.hist2[i]);
}

// One workgroup per row: resolve the threshold bin among the candidates the
// select kernel collected (a kernel boundary orders their writes before these
// reads; a device-scope fence per workgroup would write back each XCD's L2).
template <bool VEC>
__global__ __launch_bounds__(kT) void topk_refine_kernel(const float* __restrict__ scores, int64_t ld,
                                                        const int32_t* __restrict__ row_len, int k,
                                                        int32_t* __restrict__ idx, TopkWs w) {
  __shared__ SelectLds L;
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const int64_t n = row_len[row];
  if (n <= k) return;
  uint32_t c[8];
  {
    const u32x4* h = reinterpret_cast<const u32x4*>(w.hist + (size_t)row * kHistBins + 8 * t);
    const u32x4 a = h[0], b = h[1];
    c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
    c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
  }
  const Thresh th = block_threshold(c, (uint32_t)k, L.scan);
  int32_t* out = idx + (size_t)row * k;
  const uint2* gcand = w.cand + (size_t)row * w.cap;
  if (th.at <= (uint32_t)w.cap)
    refine_from_cands(L, (uint64_t)th.digit, th.above, th.at, k, out, gcand, w.hist2 + (size_t)row * kHistBins);
  else
    refine_row(L, scores + (size_t)row * ld, n, (uint64_t)th.digit, th.above, th.at, k, out, gcand, w.cap);
}

// ------------------------------------------------------------------ launchers

static int slices_for(int rows, int64_t max_len, int64_t* slice_len) {
  // Enough workgroups to cover the GPU twice, at least 2048 scores each.
  int64_t want = (512 + rows - 1) / rows;
  int64_t max_slices = (max_len + 2047) / 2048;
  if (want > max_slices) want = max_slices;
  if (want < 1) want = 1;
  int64_t len = (max_len + want - 1) / want;
  len = (len + 2047) / 2048 * 2048;
  *slice_len = len;
  return (int)((max_len + len - 1) / len);
}

static bool vec_ok(const float* scores, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(scores) % 16) == 0 && (ld % 4) == 0;
}

hipError_t launch_topk_clear(const TopkWs& w, int rows, hipStream_t st, int32_t* row_len, const int32_t* ctx_len,
                             int R) {
  const size_t total = (size_t)rows * 2 * kHistBins / 4;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 256) blocks = 256;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(topk_clear_kernel, dim3(blocks), dim3(256), 0, st, w.hist, w.ctr, rows, row_len, ctx_len, R);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float* scores, int64_t ld, const int32_t* row_len, int rows, int64_t max_len,
                            const TopkWs& w, hipStream_t st) {
  int64_t slice;
  const int ns = slices_for(rows, max_len, &slice);
  if (vec_ok(scores, ld))
    hipLaunchKernelGGL(topk_hist_kernel<true>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len, (int)slice,
                       w.hist);
  else
    hipLaunchKernelGGL(topk_hist_kernel<false>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len, (int)slice,
                       w.hist);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t ld, const int32_t* row_len, int rows, int64_t max_len,
                              int k, int32_t* idx, const TopkWs& w, hipStream_t st) {
  int64_t slice;
  const int ns = slices_for(rows, max_len < k ? k : max_len, &slice);
  if (vec_ok(scores, ld))
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len, (int)slice,
                       k, idx, w);
  else
    hipLaunchKernelGGL(topk_select_kernel<false>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len,
                       (int)slice, k, idx, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_refine_kernel<true>, dim3(rows), dim3(kT), 0, st, scores, ld, row_len, k, idx, w);
  return hipGetLastError();
}

}  // namespace dsa
