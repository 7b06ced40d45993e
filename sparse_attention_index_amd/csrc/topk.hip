// Exact top-k selection by radix select over ordered fp32 keys.
//
// "TokenSpeed Kimi K3.1", step 3: a radix top-k keeps the 2,048
// highest-scoring positions per query row; section "Reducing indexer overhead
// on AMD MI350X": one row is spread over several workgroups that share a
// histogram of score prefixes, because one workgroup per row would leave most
// of the 256 compute units idle at 4-16 decode rows.
//
// Each element is ranked by the 64-bit composite (ordered score key << 32) |
// ~position, which is unique: larger score first, then lower position. The
// top k composites are therefore a unique set.
//
// Kernels, all on one stream:
//  clear   zero each row's 2048-bin histogram and counters (a fill kernel, so
//          the sequence stays safe under stream capture);
//  hist    first digit (top 11 key bits) histogram; several workgroups per
//          row, LDS atomics then one global add per non-empty bin. The
//          decode scorer can build this histogram itself instead;
//  select  every workgroup finds the threshold bin b1 from the histogram,
//          appends positions whose bin is above b1 straight to the output
//          (wave-aggregated atomics) and collects the bin-b1 candidates;
//  refine  one workgroup per row resolves the remaining digits of the
//          composite among the candidates (or, if they overflowed their
//          buffer, over the full row) and appends the rest.
#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int kTopkThreads = 256;

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static int32_t cand_cap(int64_t max_len) {
  int64_t c = (max_len + 15) / 16;
  if (c < 4096) c = 4096;
  if (c > 65536) c = 65536;
  return (int32_t)((c + 63) / 64 * 64);
}

size_t topk_ws_bytes(int rows, int64_t max_len) {
  const size_t hist = align_up((size_t)rows * kHistBins * 4, 256);
  const size_t ctr = align_up((size_t)rows * 4 * 4, 256);
  const size_t cand = align_up((size_t)rows * cand_cap(max_len) * 8, 256);
  return hist + ctr + cand;
}

TopkWs topk_ws_carve(void* ws, int rows, int64_t max_len) {
  TopkWs w;
  char* p = static_cast<char*>(ws);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * kHistBins * 4, 256);
  w.ctr = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * 4 * 4, 256);
  w.cand = reinterpret_cast<uint2*>(p);
  w.cap = cand_cap(max_len);
  return w;
}

// ------------------------------------------------------------------ helpers

// Append `pred` lanes of the wave to a counter; returns each predicated lane's slot.
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

// Given a 2048-bin histogram h in LDS and need >= 1, find the digit d with
// count(bins > d) < need <= count(bins >= d). Block-wide; all threads get it.
struct Thresh {
  int digit;
  uint32_t above;  // count of elements in bins strictly above `digit`
};

DSA_DEV Thresh find_threshold(const uint32_t* h, uint32_t need, uint32_t* scan /*LDS [256]*/, int* res /*LDS [2]*/) {
  const int t = threadIdx.x;
  if (t == 0) {
    res[0] = 0;
    res[1] = 0;
  }
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mine += h[t * 8 + i];
  scan[t] = mine;
  __syncthreads();
  // inclusive suffix sum over threads (Hillis-Steele)
  for (int off = 1; off < kTopkThreads; off <<= 1) {
    const uint32_t v = (t + off < kTopkThreads) ? scan[t + off] : 0u;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  uint32_t above = scan[t] - mine;  // elements in bins of higher threads
  if (above < need && need <= above + mine) {
    for (int i = 7; i >= 0; --i) {
      const uint32_t c = h[t * 8 + i];
      if (above + c >= need) {
        res[0] = t * 8 + i;
        res[1] = (int)above;
        break;
      }
      above += c;
    }
  }
  __syncthreads();
  Thresh r{res[0], (uint32_t)res[1]};
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------ kernels

// Zero histograms and counters; optionally derive each row's visible length
// (position + 1) from its request's context length.
__global__ void topk_clear_kernel(uint32_t* hist, uint32_t* ctr, int rows, int32_t* row_len,
                                  const int32_t* ctx_len, int R) {
  const size_t nh = (size_t)rows * kHistBins;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = i; j < nh; j += stride) hist[j] = 0;
  for (size_t j = i; j < (size_t)rows * 4; j += stride) ctr[j] = 0;
  if (row_len)
    for (size_t j = i; j < (size_t)rows; j += stride) row_len[j] = ctx_len[j / R] - R + (int)(j % R) + 1;
}

__global__ __launch_bounds__(kTopkThreads) void topk_hist_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 const int32_t* __restrict__ row_len, int slice,
                                                                 uint32_t* __restrict__ hist) {
  __shared__ uint32_t lh[kHistBins];
  const int row = blockIdx.y;
  for (int i = threadIdx.x; i < kHistBins; i += kTopkThreads) lh[i] = 0;
  __syncthreads();
  const int64_t n = row_len[row];
  const int64_t s0 = (int64_t)blockIdx.x * slice;
  const int64_t s1 = s0 + slice < n ? s0 + slice : n;
  const float* s = scores + (size_t)row * ld;
  for (int64_t i = s0 + threadIdx.x; i < s1; i += kTopkThreads) atomicAdd(&lh[ordered_key(s[i]) >> 21], 1u);
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += kTopkThreads)
    if (lh[i]) atomicAdd(&hist[(size_t)row * kHistBins + i], lh[i]);
}

__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   const int32_t* __restrict__ row_len, int slice,
                                                                   int k, int32_t* __restrict__ idx, TopkWs w) {
  __shared__ uint32_t lh[kHistBins];
  __shared__ uint32_t scan[kTopkThreads];
  __shared__ int res[2];
  const int row = blockIdx.y;
  const int64_t n = row_len[row];
  const int64_t s0 = (int64_t)blockIdx.x * slice;
  const int64_t s1 = s0 + slice < n ? s0 + slice : n;
  int32_t* out = idx + (size_t)row * k;
  if (n <= k) {  // every visible position is selected; the rest is padding
    for (int64_t i = s0 + threadIdx.x; i < s1; i += kTopkThreads) out[i] = (int32_t)i;
    if (blockIdx.x == 0)
      for (int64_t i = n + threadIdx.x; i < k; i += kTopkThreads) out[i] = -1;
    return;
  }
  if (s0 >= n) return;  // whole workgroup idle: no barrier follows for it
  for (int i = threadIdx.x; i < kHistBins; i += kTopkThreads) lh[i] = w.hist[(size_t)row * kHistBins + i];
  __syncthreads();
  const Thresh th = find_threshold(lh, (uint32_t)k, scan, res);
  const uint32_t b1 = (uint32_t)th.digit;
  const bool keep_cands = lh[b1] <= (uint32_t)w.cap;
  uint32_t* ctr = w.ctr + (size_t)row * 4;
  uint2* cand = w.cand + (size_t)row * w.cap;
  const float* s = scores + (size_t)row * ld;
  // Iterate whole waves (uniform trip count) so the wave-level appends see every lane.
  for (int64_t base = s0; base < s1; base += kTopkThreads) {
    const int64_t i = base + threadIdx.x;
    uint32_t key = 0, bin = 0;
    const bool in = i < s1;
    if (in) {
      key = ordered_key(s[i]);
      bin = key >> 21;
    }
    const bool above = in && bin > b1;
    const uint32_t slot = wave_append(&ctr[0], above);
    if (above && slot < (uint32_t)k) out[slot] = (int32_t)i;
    if (keep_cands) {
      const bool at = in && bin == b1;
      const uint32_t cslot = wave_append(&ctr[1], at);
      if (at && cslot < (uint32_t)w.cap) cand[cslot] = make_uint2(key, (uint32_t)i);
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_refine_kernel(const float* __restrict__ scores, int64_t ld,
                                                                   const int32_t* __restrict__ row_len, int k,
                                                                   int32_t* __restrict__ idx, TopkWs w) {
  __shared__ uint32_t lh[kHistBins];
  __shared__ uint32_t scan[kTopkThreads];
  __shared__ int res[2];
  __shared__ uint32_t emitted;
  const int row = blockIdx.x;
  const int64_t n = row_len[row];
  if (n <= k) return;
  for (int i = threadIdx.x; i < kHistBins; i += kTopkThreads) lh[i] = w.hist[(size_t)row * kHistBins + i];
  if (threadIdx.x == 0) emitted = 0;
  __syncthreads();
  const Thresh th = find_threshold(lh, (uint32_t)k, scan, res);
  const uint64_t b1 = (uint64_t)th.digit;
  const uint32_t above = th.above;
  uint32_t need = (uint32_t)k - above;
  const bool from_cands = lh[b1] <= (uint32_t)w.cap;
  const uint32_t written = w.ctr[(size_t)row * 4 + 1];
  const int64_t count = from_cands ? (int64_t)(written < (uint32_t)w.cap ? written : (uint32_t)w.cap) : n;
  const uint2* cand = w.cand + (size_t)row * w.cap;
  const float* s = scores + (size_t)row * ld;
  int32_t* out = idx + (size_t)row * k;

  auto composite = [&](int64_t i) -> uint64_t {
    uint32_t key, pos;
    if (from_cands) {
      const uint2 c = cand[i];
      key = c.x;
      pos = c.y;
    } else {
      key = ordered_key(s[i]);
      pos = (uint32_t)i;
    }
    return ((uint64_t)key << 32) | (uint64_t)(~pos);
  };

  // Resolve digits below the first 11 bits: widths 11, 11, 11, 11, 9.
  uint64_t prefix = b1;
  int shift = 53;
  while (true) {
    const int width = shift < 11 ? shift : 11;
    const int lo = shift - width;
    const uint64_t mask = (1ull << width) - 1;
    for (int i = threadIdx.x; i < kHistBins; i += kTopkThreads) lh[i] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < count; i += kTopkThreads) {
      const uint64_t c = composite(i);
      if ((c >> shift) == prefix) atomicAdd(&lh[(c >> lo) & mask], 1u);
    }
    __syncthreads();
    const Thresh t = find_threshold(lh, need, scan, res);
    need -= t.above;
    const uint32_t at = lh[t.digit];
    prefix = (prefix << width) | (uint64_t)t.digit;
    shift = lo;
    __syncthreads();
    if (at == need || shift == 0) break;
  }
  // Everything in bin b1 whose composite prefix is >= the resolved prefix.
  for (int64_t base = 0; base < count; base += kTopkThreads) {
    const int64_t i = base + threadIdx.x;
    bool take = false;
    uint32_t pos = 0;
    if (i < count) {
      const uint64_t c = composite(i);
      take = (c >> 53) == b1 && (c >> shift) >= prefix;
      pos = ~(uint32_t)c;
    }
    const uint32_t slot = wave_append(&emitted, take);
    if (take && above + slot < (uint32_t)k) out[above + slot] = (int32_t)pos;
  }
}

// ------------------------------------------------------------------ launchers

static int slices_for(int rows, int64_t max_len, int64_t* slice_len) {
  // Enough workgroups to cover the GPU, but at least 4096 scores per workgroup.
  int64_t want = (1024 + rows - 1) / rows;
  int64_t max_slices = (max_len + 4095) / 4096;
  if (want > max_slices) want = max_slices;
  if (want < 1) want = 1;
  int64_t len = (max_len + want - 1) / want;
  len = (len + 255) / 256 * 256;
  if (len < 256) len = 256;
  *slice_len = len;
  return (int)((max_len + len - 1) / len);
}

hipError_t launch_topk_clear(const TopkWs& w, int rows, hipStream_t st, int32_t* row_len, const int32_t* ctx_len,
                             int R) {
  const size_t total = (size_t)rows * kHistBins;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(topk_clear_kernel, dim3(blocks), dim3(256), 0, st, w.hist, w.ctr, rows, row_len, ctx_len, R);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float* scores, int64_t ld, const int32_t* row_len, int rows, int64_t max_len,
                            const TopkWs& w, hipStream_t st) {
  int64_t slice;
  const int ns = slices_for(rows, max_len, &slice);
  hipLaunchKernelGGL(topk_hist_kernel, dim3(ns, rows), dim3(kTopkThreads), 0, st, scores, ld, row_len, (int)slice,
                     w.hist);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int64_t ld, const int32_t* row_len, int rows, int64_t max_len,
                              int k, int32_t* idx, const TopkWs& w, hipStream_t st) {
  int64_t slice;
  const int ns = slices_for(rows, max_len < k ? k : max_len, &slice);
  hipLaunchKernelGGL(topk_select_kernel, dim3(ns, rows), dim3(kTopkThreads), 0, st, scores, ld, row_len,
                     (int)slice, k, idx, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_refine_kernel, dim3(rows), dim3(kTopkThreads), 0, st, scores, ld, row_len, k, idx, w);
  return hipGetLastError();
}

}  // namespace dsa
