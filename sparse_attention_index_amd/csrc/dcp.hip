// Decode context parallelism simulated on one device: the exact top-k merge
// across W virtual shards and the log-sum-exp combine of their partial
// attention outputs.
//
// "Kimi K3.1 Pro: Day-0 Inference and RL Support with SGLang and Miles", section "Decode: DSA with decode
// context parallelism", and "vLLM Day-0 Support for Kimi K3.1 Pro", section
// "An exact top-k merge with about 10x less traffic": token p lives on shard
// p mod W; each shard takes its local top-k and sends its best C candidates;
// the k-th best of the W x C candidates is the cutoff; a shard whose C
// candidates all beat the cutoff may hold more winners and adds its whole
// local top-k; the k best of that pool are exactly the single-device top-k.
// Each shard then attends to the winners it owns, and the partial outputs are
// combined by their log-sum-exp ("TokenSpeed Kimi K3.1", section "Sharding
// long contexts with decode context parallelism").
//
// Here the shards are rows of one device's memory and the exchanges are
// plain reads. Ranking everywhere is the selection's total order: score
// descending, then position ascending, as one 64-bit composite (ordered
// score key, ~position). A candidate pool is first scattered into a
// position-indexed row (-inf outside the pool), then compacted in position
// order, so the selection kernels (which break ties by the lower index) rank
// the pool exactly as the single device ranks the row.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int kDcpThreads = 256;

static size_t a256(size_t x) { return (x + 255) / 256 * 256; }

static int64_t shard_ld(int64_t ld, int W) { return ((ld + W - 1) / W + 63) / 64 * 64; }

// Longest compacted pool of a row: every shard's whole top-k, or the row.
static int64_t comp_ld(int64_t ld, int k, int W) {
  const int64_t m = (int64_t)W * k < ld ? (int64_t)W * k : ld;
  return (m + 63) / 64 * 64;
}

struct DcpTopkWs {
  float* shard_scores;  // [rows W][lds]
  int32_t* shard_len;   // [rows W]
  int32_t* local_idx;   // [rows W][k]  shard indices of each shard's top-k
  int32_t* cand_idx;    // [rows W][C]  shard indices of each shard's top-C
  float* pool;          // [rows][ld]   position-indexed pool row (-inf outside)
  int32_t* sel;         // [rows][k]    the cutoff selection (positions)
  float* comp_score;    // [rows][cld]  the pool compacted in position order
  int32_t* comp_pos;    // [rows][cld]  their positions
  int32_t* comp_len;    // [rows]
  int32_t* comp_sel;    // [rows][k]    a selection over the compacted pool
  void* topk;           // selection workspace
};

static size_t dcp_topk_parts(int rows, int64_t ld, int k, int W, int C, DcpTopkWs* p, void* base) {
  const int64_t lds = shard_ld(ld, W);
  const int64_t cld = comp_ld(ld, k, W);
  const size_t rw = (size_t)rows * W;
  const size_t tk1 = topk_ws_bytes((int)rw, lds), tk2 = topk_ws_bytes(rows, cld);
  const size_t sizes[11] = {a256(rw * lds * 4),       a256(rw * 4),
                            a256(rw * k * 4),         a256(rw * C * 4),
                            a256((size_t)rows * ld * 4), a256((size_t)rows * k * 4),
                            a256((size_t)rows * cld * 4), a256((size_t)rows * cld * 4),
                            a256((size_t)rows * 4),    a256((size_t)rows * k * 4),
                            a256(tk1 > tk2 ? tk1 : tk2)};
  char* b = static_cast<char*>(base);
  void** slots[11] = {nullptr};
  if (p) {
    slots[0] = reinterpret_cast<void**>(&p->shard_scores);
    slots[1] = reinterpret_cast<void**>(&p->shard_len);
    slots[2] = reinterpret_cast<void**>(&p->local_idx);
    slots[3] = reinterpret_cast<void**>(&p->cand_idx);
    slots[4] = reinterpret_cast<void**>(&p->pool);
    slots[5] = reinterpret_cast<void**>(&p->sel);
    slots[6] = reinterpret_cast<void**>(&p->comp_score);
    slots[7] = reinterpret_cast<void**>(&p->comp_pos);
    slots[8] = reinterpret_cast<void**>(&p->comp_len);
    slots[9] = reinterpret_cast<void**>(&p->comp_sel);
    slots[10] = reinterpret_cast<void**>(&p->topk);
  }
  size_t off = 0;
  for (int i = 0; i < 11; ++i) {
    if (p) *slots[i] = b + off;
    off += sizes[i];
  }
  return off;
}

size_t dcp_topk_ws_bytes(int rows, int64_t ld, int k, int W, int C) {
  return dcp_topk_parts(rows, ld, k, W, C, nullptr, nullptr);
}

// Shard w of row r: positions w, w + W, ... below row_len[r], packed.
__global__ __launch_bounds__(kDcpThreads) void dcp_gather_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 const int32_t* __restrict__ row_len, int W,
                                                                 float* __restrict__ shard, int64_t lds,
                                                                 int32_t* __restrict__ shard_len) {
  const int rw = blockIdx.y;
  const int r = rw / W, w = rw % W;
  const int n = row_len[r];
  const int len = n > w ? (n - w + W - 1) / W : 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) shard_len[rw] = len;
  const int64_t i = (int64_t)blockIdx.x * kDcpThreads + threadIdx.x;
  if (i < len) shard[(size_t)rw * lds + i] = scores[(size_t)r * ld + w + (int64_t)W * i];
}

// pool[r][p] = -inf for every visible position p.
__global__ __launch_bounds__(kDcpThreads) void dcp_clear_kernel(float* __restrict__ pool, int64_t ld,
                                                                const int32_t* __restrict__ row_len) {
  const int r = blockIdx.y;
  const int64_t p = (int64_t)blockIdx.x * kDcpThreads + threadIdx.x;
  if (p < row_len[r]) pool[(size_t)r * ld + p] = -INFINITY;
}

// Put shard entries into the pool: shard w of row r contributes its top-k
// (if use_local and its resend flag is set) or its top-C.
__global__ __launch_bounds__(kDcpThreads) void dcp_scatter_kernel(const float* __restrict__ scores, int64_t ld, int W,
                                                                  int k, int C, const int32_t* __restrict__ local_idx,
                                                                  const int32_t* __restrict__ cand_idx,
                                                                  const uint8_t* __restrict__ resend,
                                                                  float* __restrict__ pool) {
  const int rw = blockIdx.x;
  const int r = rw / W, w = rw % W;
  const bool full = resend && resend[rw];
  const int32_t* src = full ? local_idx + (size_t)rw * k : cand_idx + (size_t)rw * C;
  const int n = full ? k : C;
  for (int j = threadIdx.x; j < n; j += kDcpThreads) {
    const int i = src[j];
    if (i >= 0) {
      const int64_t p = w + (int64_t)W * i;
      pool[(size_t)r * ld + p] = scores[(size_t)r * ld + p];
    }
  }
}

static constexpr int kCompThreads = 1024;

// Inclusive sum over the wave (DPP row shifts, then row broadcasts).
DSA_DEV uint32_t incl_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr 1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr 2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr 4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr 8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast 15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast 31
  return x;
}

// The pool members of row r (entries above -inf) in position order:
// comp_score / comp_pos[0 .. comp_len), one workgroup per row.
__global__ __launch_bounds__(kCompThreads) void dcp_compact_kernel(const float* __restrict__ pool, int64_t ld,
                                                                   const int32_t* __restrict__ row_len,
                                                                   float* __restrict__ comp_score,
                                                                   int32_t* __restrict__ comp_pos, int64_t cld,
                                                                   int32_t* __restrict__ comp_len) {
  __shared__ uint32_t wsum[kCompThreads / 64];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = row_len[r];
  const float* row = pool + (size_t)r * ld;
  int64_t base = 0;
  for (int64_t c0 = 0; c0 < n; c0 += 4 * kCompThreads) {
    const int64_t p0 = c0 + 4 * tid;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = p0 + e < n ? row[p0 + e] : -INFINITY;
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) cnt += v[e] > -INFINITY ? 1u : 0u;
    const uint32_t incl = incl_sum(cnt);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int w = 0; w < kCompThreads / 64; ++w) {
      const uint32_t s = wsum[w];
      before += w < wave ? s : 0u;
      total += s;
    }
    int64_t off = base + before + incl - cnt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v[e] > -INFINITY) {
        if (off < cld) {
          comp_score[(size_t)r * cld + off] = v[e];
          comp_pos[(size_t)r * cld + off] = (int32_t)(p0 + e);
        }
        ++off;
      }
    }
    base += total;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (tid == 0) comp_len[r] = (int32_t)(base < cld ? base : cld);
}

// Positions of a selection over the compacted pool.
__global__ __launch_bounds__(kDcpThreads) void dcp_map_kernel(const int32_t* __restrict__ comp_sel,
                                                              const int32_t* __restrict__ comp_pos, int64_t cld,
                                                              int rows, int k, int32_t* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * kDcpThreads + threadIdx.x;
  if (i >= (size_t)rows * k) return;
  const size_t r = i / k;
  const int j = comp_sel[i];
  out[i] = j >= 0 ? comp_pos[r * cld + j] : -1;
}

DSA_DEV uint64_t rank_of(const float* srow, int64_t p) {
  return ((uint64_t)ordered_key(srow[p]) << 32) | (uint64_t)(~(uint32_t)p);
}

// Minimum of a 64-bit value over the workgroup (every thread gets it).
DSA_DEV uint64_t block_min64(uint64_t v, uint64_t* red) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t u = __shfl_xor(v, o);
    v = u < v ? u : v;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t m = red[0];
  for (int i = 1; i < kDcpThreads / 64; ++i) m = red[i] < m ? red[i] : m;
  return m;
}

// Per row: the cutoff (the worst of the k best candidates) and each shard's
// resend flag (its C candidates all rank above the cutoff; with fewer than
// k candidates there is no cutoff and every shard that sent C resends).
__global__ __launch_bounds__(kDcpThreads) void dcp_cutoff_kernel(const float* __restrict__ scores, int64_t ld, int W,
                                                                 int k, int C, const int32_t* __restrict__ shard_len,
                                                                 const int32_t* __restrict__ cand_idx,
                                                                 const int32_t* __restrict__ sel,
                                                                 uint8_t* __restrict__ resend) {
  __shared__ uint64_t red[kDcpThreads / 64];
  const int r = blockIdx.x;
  const float* srow = scores + (size_t)r * ld;
  int ncand = 0;
  for (int w = 0; w < W; ++w) ncand += min(C, shard_len[r * W + w]);
  const bool have_cut = ncand >= k;
  uint64_t cut = 0;
  if (have_cut) {  // uniform
    uint64_t m = ~0ull;
    for (int j = threadIdx.x; j < k; j += kDcpThreads) {
      const int p = sel[(size_t)r * k + j];
      if (p >= 0) {
        const uint64_t v = rank_of(srow, p);
        m = v < m ? v : m;
      }
    }
    cut = block_min64(m, red);
  }
  for (int w = 0; w < W; ++w) {
    const int rw = r * W + w;
    if (shard_len[rw] < C) {  // sent everything it holds
      if (threadIdx.x == 0) resend[rw] = 0;
      continue;
    }
    uint64_t m = ~0ull;
    for (int j = threadIdx.x; j < C; j += kDcpThreads) {
      const int i = cand_idx[(size_t)rw * C + j];
      const uint64_t v = rank_of(srow, w + (int64_t)W * i);
      m = v < m ? v : m;
    }
    const uint64_t last = block_min64(m, red);
    if (threadIdx.x == 0) resend[rw] = (!have_cut || last > cut) ? 1 : 0;
  }
}

hipError_t launch_dcp_topk(const float* scores, int64_t ld, const int32_t* row_len, int rows, int k, int W, int C,
                           int32_t* idx, uint8_t* resend, void* ws, hipStream_t st) {
  DcpTopkWs p;
  dcp_topk_parts(rows, ld, k, W, C, &p, ws);
  const int64_t lds = shard_ld(ld, W);
  const int rw = rows * W;
  hipError_t e;
  // 1-2. shards and their local top-k and top-C
  hipLaunchKernelGGL(dcp_gather_kernel, dim3((unsigned)((lds + kDcpThreads - 1) / kDcpThreads), rw),
                     dim3(kDcpThreads), 0, st, scores, ld, row_len, W, p.shard_scores, lds, p.shard_len);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const TopkWs sw = topk_ws_carve(p.topk, rw, lds);
  if ((e = launch_topk(p.shard_scores, lds, p.shard_len, rw, lds, k, p.local_idx, sw, st)) != hipSuccess) return e;
  if ((e = launch_topk(p.shard_scores, lds, p.shard_len, rw, lds, C, p.cand_idx, sw, st)) != hipSuccess) return e;
  // 3-4. the W x C candidates, their k best, the cutoff and the resend flags
  const int64_t cld = comp_ld(ld, k, W);
  const TopkWs tw = topk_ws_carve(p.topk, rows, cld);
  const dim3 rows_grid((unsigned)((ld + kDcpThreads - 1) / kDcpThreads), rows);
  const unsigned map_grid = (unsigned)(((size_t)rows * k + kDcpThreads - 1) / kDcpThreads);
  // the k best of a scattered pool, as positions
  auto select_pool = [&](int32_t* dst) -> hipError_t {
    hipLaunchKernelGGL(dcp_compact_kernel, dim3(rows), dim3(kCompThreads), 0, st, p.pool, ld, row_len, p.comp_score,
                       p.comp_pos, cld, p.comp_len);
    hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    if ((e2 = launch_topk(p.comp_score, cld, p.comp_len, rows, cld, k, p.comp_sel, tw, st)) != hipSuccess) return e2;
    hipLaunchKernelGGL(dcp_map_kernel, dim3(map_grid), dim3(kDcpThreads), 0, st, p.comp_sel, p.comp_pos, cld, rows, k,
                       dst);
    return hipGetLastError();
  };
  hipLaunchKernelGGL(dcp_clear_kernel, rows_grid, dim3(kDcpThreads), 0, st, p.pool, ld, row_len);
  hipLaunchKernelGGL(dcp_scatter_kernel, dim3(rw), dim3(kDcpThreads), 0, st, scores, ld, W, k, C, p.local_idx,
                     p.cand_idx, (const uint8_t*)nullptr, p.pool);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = select_pool(p.sel)) != hipSuccess) return e;
  hipLaunchKernelGGL(dcp_cutoff_kernel, dim3(rows), dim3(kDcpThreads), 0, st, scores, ld, W, k, C, p.shard_len,
                     p.cand_idx, p.sel, resend);
  // 5-6. the pool with resent top-k lists, and its k best
  hipLaunchKernelGGL(dcp_clear_kernel, rows_grid, dim3(kDcpThreads), 0, st, p.pool, ld, row_len);
  hipLaunchKernelGGL(dcp_scatter_kernel, dim3(rw), dim3(kDcpThreads), 0, st, scores, ld, W, k, C, p.local_idx,
                     p.cand_idx, (const uint8_t*)resend, p.pool);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return select_pool(idx);
}

// ---------------------------------------------------------------- attention

// Shard w's part of row r is virtual row w * rows + r: its winners, its
// partial output and LSE.
size_t dcp_mla_ws_bytes(int rows, int k, int W) {
  const int vrows = W * rows;
  return a256((size_t)vrows * k * 4) + a256((size_t)vrows * 4) + a256((size_t)vrows * kMlaHeads * kV * 2) +
         a256((size_t)vrows * kMlaHeads * 4) + a256(mla_ws_bytes(vrows, k, true));
}

// The winners of row r that shard w owns (positions p with p mod W = w), in
// their order: idx_w[w * rows + r][0 .. cnt_w[w * rows + r]). One wave per
// virtual row. The row's winners are loaded 2,048 at a time, every load at
// a clamped (always valid) address so that all are in flight together;
// then, 64 at a time, a ballot marks the owned ones and each takes its slot
// from the ballot's prefix count.
__global__ __launch_bounds__(256) void dcp_owner_kernel(const int32_t* __restrict__ idx, int rows, int k, int W,
                                                       int32_t* __restrict__ idx_w, int32_t* __restrict__ cnt_w) {
  constexpr int kPerLane = 32;
  const int lane = threadIdx.x & 63;
  const int vr = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (vr >= W * rows) return;  // the whole wave
  const int w = vr / rows, r = vr - w * rows;
  const int32_t* src = idx + (size_t)r * k;
  int32_t* dst = idx_w + (size_t)vr * k;
  uint32_t cnt = 0;
  for (int c0 = 0; c0 < k; c0 += 64 * kPerLane) {
    int32_t p[kPerLane];
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) p[t] = src[min(c0 + 64 * t + lane, k - 1)];
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) {
      const bool own = c0 + 64 * t + lane < k && p[t] >= 0 && p[t] % W == w;
      const uint64_t m = __ballot(own);
      if (own)
        dst[cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = p[t];
      cnt += (uint32_t)__popcll(m);
    }
  }
  if (lane == 0) cnt_w[vr] = (int32_t)cnt;
}

// out = sum_w exp(lse_w - L) out_w, L = log sum_w exp(lse_w); one thread per
// (row, head, 4 dims).
__global__ __launch_bounds__(kDcpThreads) void dcp_combine_kernel(const uint16_t* __restrict__ out_w,
                                                                  const float* __restrict__ lse_w, int rows, int W,
                                                                  uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int r = blockIdx.y;
  const int h = threadIdx.x >> 4;
  const int d = 64 * blockIdx.x + 4 * (threadIdx.x & 15);
  const size_t rh = (size_t)r * kMlaHeads + h;
  const size_t stride_l = (size_t)rows * kMlaHeads;
  float M = -INFINITY;
  for (int w = 0; w < W; ++w) M = fmaxf(M, lse_w[w * stride_l + rh]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (M != -INFINITY) {
    for (int w = 0; w < W; ++w) {
      const float lw = lse_w[w * stride_l + rh];
      if (lw == -INFINITY) continue;
      const float f = __expf(lw - M);
      tot += f;
      const __bf16* ow = reinterpret_cast<const __bf16*>(out_w) + (w * stride_l + rh) * kV + d;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += f * (float)ow[e];
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  __bf16* o = reinterpret_cast<__bf16*>(out) + rh * kV + d;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (__bf16)(acc[e] * inv);
  if (lse && blockIdx.x == 0 && (threadIdx.x & 15) == 0) lse[rh] = tot > 0.f ? M + __logf(tot) : -INFINITY;
}

hipError_t launch_dcp_mla(const MlaArgs& a, int rows, int W, void* ws, hipStream_t st) {
  const int vrows = W * rows;
  char* b = static_cast<char*>(ws);
  int32_t* idx_w = reinterpret_cast<int32_t*>(b);
  b += a256((size_t)vrows * a.k * 4);
  int32_t* cnt_w = reinterpret_cast<int32_t*>(b);
  b += a256((size_t)vrows * 4);
  uint16_t* out_w = reinterpret_cast<uint16_t*>(b);
  b += a256((size_t)vrows * kMlaHeads * kV * 2);
  float* lse_w = reinterpret_cast<float*>(b);
  b += a256((size_t)vrows * kMlaHeads * 4);
  void* mla_ws = b;
  hipLaunchKernelGGL(dcp_owner_kernel, dim3((unsigned)((vrows + 3) / 4)), dim3(256), 0, st, a.idx, rows, a.k, W,
                     idx_w, cnt_w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // every shard's partial attention over the winners it owns, in one launch
  // over the virtual rows (each takes its query and request from row r)
  MlaArgs s = a;
  s.idx = idx_w;
  s.slots = nullptr;
  s.out = out_w;
  s.lse = lse_w;
  s.q_rows = rows;
  s.nvalid = cnt_w;
  if ((e = launch_sparse_mla(s, vrows, true, mla_ws, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(dcp_combine_kernel, dim3(kV / 64, rows), dim3(kDcpThreads), 0, st, out_w, lse_w, rows, W,
                     a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
