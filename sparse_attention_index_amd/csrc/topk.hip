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
//          (a slice that overflowed its region is read again from the row)
//          and radix-selects the k largest composites. The answer is exact
//          whenever at least k candidates were collected, because every
//          element of the top k is then >= T; if fewer than k or more than
//          fit arrived, the workgroup selects over the whole row instead.
//          The sample only decides the speed, never the result.
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace dsa {

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

// Workspace: per (row, slice) count and largest key, per row threshold, then
// the candidate regions.
size_t topk_ws_bytes(int rows, int64_t max_len) {
  (void)max_len;
  return 2 * align_up((size_t)rows * kMaxSlices * 4, 256) + align_up((size_t)rows * 4, 256) +
         align_up((size_t)rows * cand_cap(rows) * 8, 256);
}

TopkWs topk_ws_carve(void* ws, int rows, int64_t max_len) {
  (void)max_len;
  TopkWs w;
  char* p = static_cast<char*>(ws);
  w.cnt = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * kMaxSlices * 4, 256);
  w.tmax = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * kMaxSlices * 4, 256);
  w.thr = reinterpret_cast<uint32_t*>(p);
  p += align_up((size_t)rows * 4, 256);
  w.cand = reinterpret_cast<uint2*>(p);
  w.cap = cand_cap(rows);
  return w;
}

// ------------------------------------------------------------------ final

struct FinalLds {
  SelectLds s;
  uint32_t off[kMaxSlices + 1];  // each slice's first survivor in the row's run; the total last
  uint32_t cnt[kMaxSlices];      // each slice's survivors
  uint32_t fill;                 // survivors of an overflowed slice found again so far
  uint32_t kmax;                 // the row's largest key
  uint2 elems[kFinalLds];
};

// ------------------------------------------------------------------ short rows

// Rows of at most kShortMax scores: one workgroup of kTF threads per row
// holds the whole row in registers (score 4096 q + 4 t + e is x[4 q + e] of
// thread t), keeps every score >= T in LDS and selects the k largest there:
// one kernel, no global round trip. The samples and the row are loaded
// together, so the threshold is found while the row is in flight.
static constexpr int kShortPer = 40;                // scores per thread
static constexpr int kShortMax = kTF * kShortPer;   // 40,960

struct ShortLds {
  SelectLds f;
  uint32_t cnt;
  uint32_t wmax[kTF / 64];
  uint32_t wmin[kTF / 64];
  int32_t tbl[kShortMax / kBlock];  // page ids of the row's request (when slots are emitted)
  uint2 elems[kFinalLds + 1];       // survivors, plus one spare entry taking overflow writes
};

template <bool VEC>
__global__ __launch_bounds__(kTF) void topk_short_kernel(const float* __restrict__ scores, int64_t ld,
                                                       int32_t* __restrict__ row_len, const int32_t* ctx_len, int R,
                                                       int k, int32_t* __restrict__ idx, SlotOut so) {
  constexpr int G = kShortPer / 4;  // 16-byte groups per thread
  __shared__ ShortLds L;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = blockIdx.x;
  const int n = (int)visible_len(row_len, ctx_len, R, row, ld);  // <= ld <= kShortMax
  if (ctx_len && t == 0) row_len[row] = n;  // published for the caller
  int32_t* out = idx + (size_t)row * k;
  int32_t* slots = so.slots ? so.slots + (size_t)row * k : nullptr;
  const int32_t* table = so.slots ? so.block_table + (size_t)(row / R) * so.max_blocks : nullptr;
  if (n <= k) {  // every visible position is selected; the rest is padding
    for (int i = t; i < k; i += kTF) {
      out[i] = i < n ? i : -1;
      if (slots) slots[i] = i < n && (i >> 6) < so.max_blocks ? table[i >> 6] * kBlock + (i & 63) : -1;
    }
    return;
  }
  // the request's page ids, loaded first so that waiting for them waits for nothing else
  int32_t tv = 0;
  const int npages = (n + kBlock - 1) / kBlock;
  if (slots && t < npages) tv = t < so.max_blocks ? table[t] : -1;
  const float* s = scores + (size_t)row * ld;
  uint32_t skey[kSample / kTF];
  sample_load<kTF>(s, n, skey);
  // The row through a buffer descriptor of n scores (one VGPR offset per
  // lane); groups that start past n are not loaded.
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s), (short)0, 4 * n, 0x00020000);
  float x[kShortPer];
#pragma unroll
  for (int q = 0; q < G; ++q) {
    if (4096 * q < n) {  // uniform
      if (VEC) {
        const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * t, 16384 * q, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[4 * q + e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, 16 * t + 4 * e, 16384 * q, 0));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = __builtin_nanf("");
    }
  }
  if (t == 0) L.cnt = 0;
  if (slots && t < npages) L.tbl[t] = tv;  // read after the barriers below
  lds_barrier();  // the counter is cleared before any wave reserves (the row loads stay in flight)
  const uint32_t T = sample_select<kTF>(skey, n, k, L.f.hist, L.f.scan);
  const float Tf = key_threshold_float(T);
  // The group holding position n - 1 (index qb): NaN past n, and with
  // 16-byte loads the scores of a partial vector read again one by one (the
  // buffer load of a vector that crosses the end may return zeros). NaN is
  // never kept.
  {
    const int qb = (n - 1) / 4096;  // uniform
    float y[4];
    bool past[4], reread[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4096 * qb + 4 * t + e;
      past[e] = i >= n;
      reread[e] = VEC && !past[e] && i >= (n & ~3);
      y[e] = reread[e] ? s[i] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (q == qb) {  // uniform
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] = past[e] ? __builtin_nanf("") : (reread[e] ? y[e] : x[4 * q + e]);
      }
    }
  }
  // survivors -> LDS as (score bits, position): one reservation per wave;
  // slots past the buffer all land on its spare last entry. The row's
  // largest score bounds the survivors from above, and the larger of T and
  // its smallest from below (rows that keep everything have T = 0: a bound
  // at 0 would put all of them in the first radix step's top bin).
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) {  // NaN operands are ignored
    mx = fmaxf(mx, x[j]);
    mn = fminf(mn, x[j]);
  }
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) mine += (uint32_t)(x[j] >= Tf);
  uint32_t total;
  const uint32_t pre = wave_prefix_small<6>(mine, total);
  uint32_t slot = wave_reserve(&L.cnt, total) + pre;
  uint32_t pbase = (uint32_t)(4 * t);
  float tf = Tf;
  // keeps the compiler from precomputing every position, and makes the
  // comparisons again here rather than holding forty masks from the count
  // above in scalar registers (which spill)
  asm volatile("" : "+v"(pbase), "+v"(tf));
#pragma unroll
  for (int j = 0; j < kShortPer; ++j) {
    const bool kp = x[j] >= tf;
    if (kp)
      L.elems[slot < (uint32_t)kFinalLds ? slot : (uint32_t)kFinalLds] =
          make_uint2(__float_as_uint(x[j]), pbase + (uint32_t)(4096 * (j >> 2) + (j & 3)));
    slot += kp;
  }
  const uint32_t wm = wave_max32(ordered_key(mx));
  const uint32_t wn = ~wave_max32(~ordered_key(mn));
  if (lane == 0) {
    L.wmax[wave] = wm;
    L.wmin[wave] = wn;
  }
  __syncthreads();
  const uint32_t count = L.cnt;
  const uint32_t kmax = wave_max32(lane < kTF / 64 ? L.wmax[lane] : 0u);
  const uint32_t kmin = ~wave_max32(lane < kTF / 64 ? ~L.wmin[lane] : 0u);
  const Emit emit{out, slots, L.tbl};
  if (count >= (uint32_t)k && count <= (uint32_t)kFinalLds)
    select_top(
        L.f, count, k, emit,
        [&](int64_t i) { return composite(ordered_key(__uint_as_float(L.elems[i].x)), L.elems[i].y); }, true,
        (uint64_t)(T > kmin ? T : kmin) << 32, ((uint64_t)kmax << 32) | 0xffffffffull);
  else  // the sample missed: select over the whole row
    select_top(L.f, n, k, emit, [&](int64_t i) { return composite(ordered_key(s[i]), (uint32_t)i); });
}

// ------------------------------------------------------------------ long rows

// Grid (slices, rows), kT threads: workgroup x streams its slice of the row
// (16 scores per lane and step, the next step in flight) and writes every
// score >= T, as (ordered key, position), to its own region of the row's
// candidate buffer; then its true count, its largest key and (slice 0) T go
// to slots of its own: no global atomics, nothing to clear first. The first
// two steps are issued once the samples have arrived, so the threshold is
// found while they are in flight.
static constexpr int kT = 256;

struct SliceLds {
  ScanLds<kT> scan;
  uint32_t hist[kHistBins];
  uint32_t cnt;
  uint32_t wmax[kT / 64];
};

template <bool VEC>
__global__ __launch_bounds__(kT) void topk_slice_kernel(const float* __restrict__ scores, int64_t ld,
                                                       int32_t* __restrict__ row_len, const int32_t* ctx_len, int R,
                                                       int slice, int k, TopkWs w) {
  __shared__ SliceLds L;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = blockIdx.y;
  const int64_t n = visible_len(row_len, ctx_len, R, row, ld);
  if (ctx_len && blockIdx.x == 0 && t == 0) row_len[row] = (int32_t)n;  // published for the caller
  if (n <= k) return;  // the final kernel emits every position
  const float* s = scores + (size_t)row * ld;
  const int64_t s0 = (int64_t)blockIdx.x * slice;
  const int64_t s1 = s0 + slice < n ? s0 + slice : n;
  const uint32_t sub = (uint32_t)(w.cap / gridDim.x);  // this slice's share of the row's buffer
  uint2* gcand = w.cand + (size_t)row * w.cap + (size_t)blockIdx.x * sub;

  // Step of 4096 scores at base: lane element (q, e) is position
  // base + 1024 wave + 4 lane + 256 q + e, read through a buffer descriptor
  // of the slice (past its end the loads return 0 and no branch is needed,
  // so the compiler keeps several steps' loads in flight).
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(s + s0), (short)0,
                                                      (int)(4 * (s1 > s0 ? s1 - s0 : 0)), 0x00020000);
  auto load_step = [&](int64_t base, float (&v)[16]) {
    const int off = (int)(4 * (base - s0)) + 16 * (256 * wave + lane);
    if (VEC) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 1024 * q, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, off + 4 * (j & 3), 1024 * (j >> 2), 0));
    }
  };
  // The samples travel alone (the slice loads of every workgroup would delay
  // them); the first two steps of the slice are in flight while the
  // threshold is computed.
  uint32_t skey[kSample / kT];
  sample_load<kT>(s, n, skey);
  wait_vmcnt<0>();
  // Two step buffers in turn, loaded unconditionally (past the slice the
  // descriptor returns zeros that no test reads): with no branch around a
  // load, the compiler's wait before a step is for that step's loads only,
  // and the other buffer's stay in flight behind it (a register copy from a
  // `next` buffer would wait for every load).
  float bufa[16], bufb[16];
  load_step(s0, bufa);
  load_step(s0 + 4096, bufb);
  if (t == 0) L.cnt = 0;
  lds_barrier();  // the counter is cleared before any wave reserves (the loads stay in flight)
  const uint32_t T = sample_select<kT>(skey, n, k, L.hist, L.scan);
  const float Tf = key_threshold_float(T);

  float mx = -INFINITY;
  auto step = [&](int64_t base, float (&cur)[16]) {
    const bool whole = base + 4096 <= s1;  // uniform: no position test needed
    const int64_t wbase = base + 1024 * wave + 4 * lane;
    if (VEC && !whole && (s1 & 3)) {
      // The 16-byte load of the vector that crosses the slice's end (only
      // the row's last slice ends off a multiple of 4) may return zeros for
      // its in-range scores too: the one lane holding it reads them again
      // one by one.
      const int64_t vs = s1 & ~(int64_t)3;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (wbase + 256 * q == vs) {
#pragma unroll
          for (int e = 0; e < 3; ++e)
            if (vs + e < s1) cur[4 * q + e] = s[vs + e];
        }
      }
    }
    uint32_t cmask = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool in = whole || wbase + 256 * (j >> 2) + (j & 3) < s1;
      cmask |= (uint32_t)(in && cur[j] >= Tf) << j;
      if (in) mx = fmaxf(mx, cur[j]);
    }
    uint32_t tc;
    const uint32_t pc = wave_prefix_small<5>((uint32_t)__popc(cmask), tc);
    uint32_t slot = wave_reserve(&L.cnt, tc) + pc;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (cmask & (1u << j)) {
        if (slot < sub) gcand[slot] = make_uint2(ordered_key(cur[j]), (uint32_t)(wbase + 256 * (j >> 2) + (j & 3)));
        ++slot;
      }
    }
  };
  for (int64_t base = s0; base < s1; base += 8192) {
    step(base, bufa);
    load_step(base + 8192, bufa);
    if (base + 4096 < s1) step(base + 4096, bufb);  // uniform
    load_step(base + 12288, bufb);
  }
  const uint32_t wm = wave_max32(ordered_key(mx));
  if (lane == 0) L.wmax[wave] = wm;
  __syncthreads();
  if (t == 0) {
    // the true count, also when it overflowed the region: the final kernel
    // then selects over the whole row
    w.cnt[(size_t)row * kMaxSlices + blockIdx.x] = L.cnt;
    w.tmax[(size_t)row * kMaxSlices + blockIdx.x] = max(max(L.wmax[0], L.wmax[1]), max(L.wmax[2], L.wmax[3]));
    if (blockIdx.x == 0) w.thr[row] = T;
  }
}

// One workgroup per row gathers the slices' survivors (a kernel boundary
// orders the slice workgroups' writes before these reads; a device-scope fence
// per workgroup would write back each XCD's L2). A slice whose survivors
// overflowed its region (they cluster where the row's high scores do, for
// instance among the most recent positions) is read again from the score row
// with the slice pass's own test, so the run holds every survivor either way.
// Every survivor lies in [T << 32, (largest key << 32) | ~0], which saves
// select_top a pass.
template <bool VEC>
__global__ __launch_bounds__(kTF) void topk_final_kernel(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ row_len, int R, int slices,
                                                       int slice, int k, int32_t* __restrict__ idx, TopkWs w,
                                                       SlotOut so) {
  __shared__ FinalLds L;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = blockIdx.x;
  const int64_t n = visible_len(row_len, nullptr, 1, row, ld);  // published by the slice pass
  int32_t* out = idx + (size_t)row * k;
  if (n <= k) {  // every visible position is selected; the rest is padding
    emit_all_positions(row, R, n, k, out, so);
    return;
  }
  const Emit emit{out, nullptr, nullptr};
  // slices' true counts and their offsets in LDS: lane t of wave 0 owns slice t
  const uint32_t sub = (uint32_t)(w.cap / slices);
  if (t < 64) {
    const uint32_t c = t < slices ? w.cnt[(size_t)row * kMaxSlices + t] : 0u;
    const uint32_t km = t < slices ? w.tmax[(size_t)row * kMaxSlices + t] : 0u;
    const uint32_t incl = wave_incl_sum(c);
    const uint32_t kmax = wave_max32(km);
    if (t < slices) {
      L.off[t] = incl - c;
      L.cnt[t] = c;
    }
    if (t == 63) L.off[slices] = incl;
    if (t == 0) {
      L.kmax = kmax;
      L.fill = 0;
    }
  }
  const uint32_t T = w.thr[row];
  const float Tf = key_threshold_float(T);
  __syncthreads();
  const uint32_t count = L.off[slices];
  const float* s = scores + (size_t)row * ld;
  if (count >= (uint32_t)k && count <= (uint32_t)kFinalLds) {
    // regions that hold their slice's survivors: groups of wps waves (one
    // wave when there are 16 slices or more, all 16 for a single slice) copy
    // slices g, g + groups, ..., four loads in flight per lane
    const uint2* regions = w.cand + (size_t)row * w.cap;
    constexpr int kWaves = kTF / 64;
    const int wps = slices >= kWaves ? 1 : kWaves / slices;  // waves per slice
    const int groups = kWaves / wps;
    const int gw = wave / wps;                       // this wave's group
    const uint32_t gl = 64 * (wave % wps) + lane;    // its lane within the group
    const uint32_t gsz = 64 * wps;
    for (int r = gw; gw < groups && r < slices; r += groups) {
      const uint32_t o = L.off[r], cr = L.cnt[r];
      if (cr > sub) continue;  // read again below (uniform over the group)
      for (uint32_t j0 = 0; j0 < cr; j0 += 4 * gsz) {
        uint2 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t j = j0 + gsz * u + gl;
          v[u] = j < cr ? regions[(size_t)r * sub + j] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t j = j0 + gsz * u + gl;
          if (j < cr) L.elems[o + j] = v[u];
        }
      }
    }
    // overflowed slices: the whole workgroup streams the slice again (16
    // scores per thread and step) and keeps score >= Tf, as the slice pass
    // did; at most cr survivors are written
    for (int r = 0; r < slices; ++r) {
      const uint32_t cr = L.cnt[r];
      if (cr <= sub) continue;  // uniform
      const uint32_t o = L.off[r];
      const int64_t a0 = (int64_t)r * slice;
      const int64_t a1 = a0 + slice < n ? a0 + slice : n;
      for (int64_t base = a0; base < a1; base += 16 * kTF) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t p = base + 4 * kTF * q + 4 * t;
          if (VEC && p + 3 < a1) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(s + p);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = p + e < a1 ? s[p + e] : __builtin_nanf("");
          }
        }
        uint32_t cmask = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) cmask |= (uint32_t)(v[j] >= Tf) << j;  // NaN is never kept
        uint32_t tc;
        const uint32_t pc = wave_prefix_small<5>((uint32_t)__popc(cmask), tc);
        uint32_t slot = wave_reserve(&L.fill, tc) + pc;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (cmask & (1u << j)) {
            const int64_t p = base + 4 * kTF * (j >> 2) + 4 * t + (j & 3);
            if (slot < cr) L.elems[o + slot] = make_uint2(ordered_key(v[j]), (uint32_t)p);
            ++slot;
          }
        }
      }
      __syncthreads();  // every wave has reserved from the counter
      if (t == 0) L.fill = 0;
      __syncthreads();
    }
    __syncthreads();
    select_top(
        L.s, count, k, emit, [&](int64_t i) { return composite(L.elems[i].x, L.elems[i].y); }, true,
        (uint64_t)T << 32, ((uint64_t)L.kmax << 32) | 0xffffffffull);
  } else {  // the sample missed: select over the whole row
    select_top(L.s, n, k, emit, [&](int64_t i) { return composite(ordered_key(s[i]), (uint32_t)i); });
  }
  if (so.slots) {
    __syncthreads();  // the selection is written (workgroup-visible)
    emit_slots(row, R, k, out, so);
  }
}

// ------------------------------------------------------------------ launcher

static bool vec_ok(const float* scores, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(scores) % 16) == 0 && (ld % 4) == 0;
}

hipError_t launch_topk(const float* scores, int64_t ld, int32_t* row_len, int rows, int64_t max_len, int k,
                       int32_t* idx, const TopkWs& w, hipStream_t st, const int32_t* ctx_len, int R,
                       const SlotOut& so) {
  const bool vec = vec_ok(scores, ld);
  if (max_len <= kShortMax) {
    if (vec)
      hipLaunchKernelGGL(topk_short_kernel<true>, dim3(rows), dim3(kTF), 0, st, scores, ld, row_len, ctx_len, R, k,
                         idx, so);
    else
      hipLaunchKernelGGL(topk_short_kernel<false>, dim3(rows), dim3(kTF), 0, st, scores, ld, row_len, ctx_len, R, k,
                         idx, so);
    return hipGetLastError();
  }
  // Slices: enough workgroups to cover the GPU twice, at least 4096 scores
  // and at most kMaxSlices workgroups per row.
  int64_t want = (512 + rows - 1) / rows;
  const int64_t max_slices = (max_len + 4095) / 4096;
  if (want > max_slices) want = max_slices;
  if (want > kMaxSlices) want = kMaxSlices;
  if (want < 1) want = 1;
  int64_t slice = (max_len + want - 1) / want;
  slice = (slice + 4095) / 4096 * 4096;
  const int ns = (int)((max_len + slice - 1) / slice);
  if (vec)
    hipLaunchKernelGGL(topk_slice_kernel<true>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len, ctx_len, R,
                       (int)slice, k, w);
  else
    hipLaunchKernelGGL(topk_slice_kernel<false>, dim3(ns, rows), dim3(kT), 0, st, scores, ld, row_len, ctx_len, R,
                       (int)slice, k, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (vec)
    hipLaunchKernelGGL(topk_final_kernel<true>, dim3(rows), dim3(kTF), 0, st, scores, ld, row_len, R, ns, (int)slice,
                       k, idx, w, so);
  else
    hipLaunchKernelGGL(topk_final_kernel<false>, dim3(rows), dim3(kTF), 0, st, scores, ld, row_len, R, ns,
                       (int)slice, k, idx, w, so);
  return hipGetLastError();
}

}  // namespace dsa
