// Lightning-indexer scoring on gfx950 MFMA.
//
// score(row, s) = sum_h w[row][h] * ReLU(q[row][h] . key_s) * key_scale[s]
// ("vLLM Day-0 Support for Kimi K3.1 Pro", section "What Kimi K3.1 Pro
// changes": 32 heads x 128 dims over one 132-byte FP8 key per token).
//
// Work decomposition. A workgroup (4 waves) owns a group of 4*RPW query rows
// of one request (wave w: rows w*RPW .. w*RPW+RPW-1) and walks a strided set
// of that request's 64-token pages. Each page's 8 KB of keys and 256 B of
// scales are read from HBM once, staged in LDS and used by all the group's
// rows ("TokenSpeed Kimi K3.1", section "Reducing indexer overhead on AMD
// MI350X": each key is loaded once for all of a request's verification
// rows). The workgroup's page ids are read from the block table once, up
// front, into LDS. Requests get workgroups in proportion to their pages
// (wg_range, computed in the kernel from ctx_len), so ragged requests
// finish together ("vLLM Day-0 Support for Kimi K3.1 Pro", section "Fused
// low-latency decode for DSA layers": a key-balanced scorer).
//
// Streaming. The page copies go from HBM straight into a ring of kRing LDS
// slots (global_load_lds, no VGPR staging) and kRing - 1 pages stay in
// flight. Waves 0-2 each issue a third of every page's copies and wait on
// their own vmcnt; their scores go to LDS, and wave 3 stores all rows'
// scores. A wave that issues both loads and stores can only wait for all of
// its outstanding operations, so keeping the copying waves free of global
// stores keeps their vmcnt an exact count of copies and the waits never
// drain the ring. One barrier per page hands a full slot to the waves and
// the slot they finished back to the copiers. Workgroups of four waves take
// one wave slot per SIMD, so several fit a CU and overlap each other's MFMA
// and VALU work; the copy and store duties are spread so that no wave (and
// no SIMD) carries much more than the others.
// Score stores use buffer descriptors sized to each row's visible prefix:
// the hardware drops stores past it, which applies the causal mask without
// branches. In the filtered decode nothing is stored but the candidates:
// each wave compares its own rows' scores with their thresholds as it
// reduces them and appends the few that pass to its workgroup's region of
// the row's buffer.
//
// The dot products run on v_mfma_f32_32x32x64_f8f6f4 (the scaled form for
// MXFP4 keys) with the raw key bytes as the B operand (no conversion).
// Queries enter as E4M3:
//  * E4M3 queries (prefill chunks) are used as they are, their row scale
//    applied after the head reduction;
//  * bf16 queries are split into two E4M3 terms, q * 2^e = hi + lo,
//    with a power-of-two scale 2^e per (row, head) that puts the head's
//    largest magnitude in (224, 448]. A bf16 value has 8 significant bits
//    and each E4M3 term carries 4, so hi + lo reproduces it exactly except
//    for elements more than ~2^10 below the head maximum, whose residual
//    falls under E4M3's subnormal step (error below 2^-10 of that step);
//    products E4M3 x E4M3 are exact and accumulate in fp32. The two terms
//    cost two MFMAs, the same issue time as one bf16 MFMA of the same shape,
//    and the keys need no widening.
// The 32x32 output tile puts 16 heads of one key in each lane, so the
// head-weighted ReLU reduction is 16 in-lane max+fma steps plus one
// permlane32 swap between the lane halves. With one or two rows per wave the
// MFMAs of each 32-key half are interleaved with the epilogue of the half
// before it. 2^-e, the key scale and the
// query row scale are positive and are applied after the ReLU.
//
// K (the 128 key dims) is permuted identically in both operands: lane half
// g of a 32x32x64 step s holds dims 64g + 32s + [0, 32).
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "query.h"
#include "select.h"

namespace dsa {

static constexpr int kKeyBytes = kBlock * kIdxDim;  // one page of keys, 8 KB
static constexpr int kF4KeyBytes = kBlock * kIdxDim / 2;  // one page of MXFP4 keys, 4 KB
static constexpr int kF4Copies = kF4KeyBytes / 1024 + 1;  // 4 key copies + 1 scale copy
static constexpr int kRing = 4;                     // LDS page slots per workgroup
// Pages one workgroup walks at most (its page ids are staged in LDS): 4,096
// for the 16-row prefill variant, whose registers already hold it to two
// workgroups per CU, so that a 256K-token chunk still takes one round of
// them; 1,024 for one row per wave, so that four workgroups fit a CU's LDS;
// 2,048 for the others, where more would cost a resident workgroup.
template <int RPW>
constexpr int max_wg_pages() {
  return RPW == 4 ? 4096 : (RPW == 1 ? 1024 : 2048);
}
// Waves per SIMD the register allocation aims at: four for the filtered
// decode with one row per wave and FP8 keys (128 registers: four
// workgroups per CU, measured 3-4% faster than three), two otherwise.
template <int RPW, bool QFP8, bool KF4, bool FILT>
constexpr int score_waves_per_eu() {
  return FILT && RPW == 1 && !KF4 ? 4 : 2;
}
static constexpr int kThreads = 256;                // 4 waves
static constexpr int kCopies = kKeyBytes / 1024 + 1;  // copy instructions per page (keys + scales)
static constexpr int kCopiers = 3;                  // waves that issue copies
static constexpr int kCopiesPerWave = kCopies / kCopiers;
static_assert(kCopies % kCopiers == 0, "copies split evenly");

// LDS position of 16-byte chunk j of key n within a staged page: rows of
// 128 B with the chunk index XOR-swizzled by (n >> 1) & 7 so that the 16
// lanes of each read phase hit distinct banks.
DSA_DEV int key_chunk_off(int n, int j) { return n * kIdxDim + ((j ^ ((n >> 1) & 7)) << 4); }

// Wave priority from the workgroup's progress: 3 over its first quarter of
// pages down to 0 over its last. Several workgroups share each SIMD and the
// oldest wave wins ties, so without this the first workgroup placed on a CU
// races ahead and the last one finishes the kernel alone; with it, the
// workgroups that lag get issued first and all finish at about the same time.
DSA_DEV void set_progress_priority(int i, int n) {
  const int lvl = (4 * (n - i)) / (n + 1);
  if (lvl >= 3) __builtin_amdgcn_s_setprio(3);
  else if (lvl == 2) __builtin_amdgcn_s_setprio(2);
  else if (lvl == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Byte offset past every row's visible prefix: buffer stores there are dropped.
static constexpr uint32_t kPastEnd = 0x80000000u;

// Roles of the waves: every wave scores RPW rows and writes its scores to
// LDS; waves 0-2 also move the pages into LDS, wave 3 stores the scores.
enum WaveRole { kCopier, kFlusher };

template <int RPW, bool QFP8, bool KF4, bool FILT>
__global__ __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(score_waves_per_eu<RPW, QFP8, KF4, FILT>()))) void score_kernel(ScoreArgs a,
                                                                                                       int B) {
  constexpr int ROWS = 4 * RPW;
  constexpr int NT = QFP8 ? 1 : 2;  // E4M3 terms per query value
  constexpr int LAG = 2;             // a page's scores are complete two barriers later
  constexpr int PAGE = KF4 ? kF4KeyBytes : kKeyBytes;
  __shared__ __attribute__((aligned(16))) uint8_t key_s[kRing][PAGE];
  __shared__ __attribute__((aligned(16))) float ks_s[kRing][kBlock];  // fp32 scales, or 4 E8M0 per key
  __shared__ int32_t tbl_s[max_wg_pages<RPW>()];
  __shared__ __attribute__((aligned(16))) float w_s[ROWS][kIdxHeads];
  __shared__ float sc_s[LAG + 1][ROWS][kBlock];  // scores of the group's rows, by page

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 5;   // lane half
  const int n = lane & 31;   // A row (head) / B and D column (key)
  // this workgroup's request and its place among that request's workgroups
  // (workgroups are handed out in proportion to the requests' pages)
  const WgRange wgr = wg_range(a.ctx_len, B, gridDim.x, blockIdx.x, -1);
  const int b = wgr.b;
  const int R = a.R;
  const int r0 = blockIdx.z * ROWS;           // first row of the group within the request
  const int nr = min(ROWS, R - r0);           // rows of the group that exist
  const int L = a.ctx_len[b];
  const int pos0 = L - R + r0;                // position of the group's first row
  const int blk_lim = ((pos0 + nr - 1) >> 6) + 1;  // pages any row of the group sees
  const size_t row0 = (size_t)b * R + r0;

  // this workgroup's pages: jx, jx + stride, ... below blk_lim
  const int jx = blockIdx.x - wgr.first;
  const int stride = wgr.count;
  const int n_my = blk_lim > jx ? (blk_lim - jx + stride - 1) / stride : 0;
  const int wr0 = wave * RPW;

  // Score stores go through one buffer descriptor per row whose size is the
  // row's visible prefix (positions 0 .. pos): the hardware drops any store
  // at or past it, which is the causal mask, and lanes that hold no row's
  // total store at an offset past every prefix. Stores are branch-free.
  auto row_rsrc = [&](int gr) {
    const int gv = min(gr, nr - 1);
    const int bytes = gr < nr ? 4 * (pos0 + gr + 1) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(a.scores + (row0 + gv) * a.ld, (short)0, bytes, 0x00020000);
  };

  // Copy j of a page moves LDS chunks 64j .. 64j+63 of the page's swizzled
  // layout: lane l fetches the global chunk that belongs at LDS chunk 64j + l.
  // The last copy moves the page's 64 scales. Wave w issues copies
  // w*kCopiesPerWave .. w*kCopiesPerWave + kCopiesPerWave - 1.
  // MXFP4 pages: 4 copies of 1 KB (16-byte chunks of 64-byte key rows,
  // chunk c of key r at position c ^ ((r >> 2) & 3)) and one of the 64 keys'
  // E8M0 words; waves 0 and 1 issue two key copies each, wave 2 the scales.
  // Page bases are wave-uniform (scalar registers); lanes add 32-bit offsets.
  auto issue = [&](int i) {
    const int slot = i % kRing;
    const size_t page = (uint32_t)__builtin_amdgcn_readfirstlane(tbl_s[i]);
    if constexpr (KF4) {
      const uint8_t* pg = a.key_fp4 + page * kF4KeyBytes;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * wave + jj;  // wave-uniform
        if (j < kF4Copies - 1) {
          const int c = 64 * j + lane;
          const int key = c >> 2;
          copy16_to_lds_at(pg, (uint32_t)(key * (kIdxDim / 2) + (((c & 3) ^ ((key >> 2) & 3)) << 4)),
                           key_s[slot] + 1024 * j);
        } else if (j == kF4Copies - 1) {
          copy4_to_lds_at(a.key_e8m0 + page * kBlock * 4, (uint32_t)lane * 4, ks_s[slot]);
        }
      }
      return;
    }
    const uint8_t* pg = a.key_fp8 + page * kKeyBytes;
#pragma unroll
    for (int jj = 0; jj < kCopiesPerWave; ++jj) {
      const int j = wave * kCopiesPerWave + jj;
      if (j < kCopies - 1) {
        const int c = 64 * j + lane;
        const int key = c >> 3;
        copy16_to_lds_at(pg, (uint32_t)(key * kIdxDim + (((c & 7) ^ ((key >> 1) & 7)) << 4)), key_s[slot] + 1024 * j);
      } else {
        copy4_to_lds_at(a.key_scale + page * kBlock, (uint32_t)lane * 4, ks_s[slot]);
      }
    }
  };

  // ---- prologue. The query rows and head weights are loaded first and the
  // page table second, so that both loads are in flight together; one wait
  // takes all of them. The copiers then put the first pages in flight before
  // the queries are converted, so the conversion overlaps their latency.
  // From here on a copier's only vector-memory operations are its copies.
  QueryRaw<QFP8, KF4> qraw[RPW];
  uint32_t wbits[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const size_t row = row0 + min(wr0 + rr, nr - 1);  // clamp: rows past the group reuse a valid row, never written
    fetch_query<QFP8, KF4>(a, row, n, g, qraw[rr]);
    wbits[rr] = a.w[row * kIdxHeads + n];
  }
  // filtered decode: the threshold of each of the wave's rows, loaded with the queries
  float thr_w[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) thr_w[rr] = FILT ? a.thr[row0 + min(wr0 + rr, nr - 1)] : 0.f;
  {
    const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
    for (int i = tid; i < n_my; i += kThreads) tbl_s[i] = table[jx + i * stride];
  }
  wait_vmcnt<0>();
  __syncthreads();  // tbl_s ready
  if (wave < kCopiers) {
    for (int i = 0; i < kRing - 1 && i < n_my; ++i) issue(i);
  }
  i32x8 A[RPW][NT][2];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    hold_query(qraw[rr]);
    const float head_scale = finish_query(qraw[rr], A[rr]);
    // head weights with the head's scale folded in: w_s[row][head]
    if (g == 0) w_s[wr0 + rr][n] = __uint_as_float(wbits[rr] << 16) * head_scale;
  }
  __syncthreads();  // w_s ready
  // the 16 heads this lane reduces (rows 8*(i/4) + 4g + i%4 of the 32x32 tile);
  // kept in VGPRs for one row per wave, read from LDS otherwise
  float wv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) wv[i] = w_s[wr0][8 * (i >> 2) + 4 * g + (i & 3)];

  // filtered decode: the candidates each of the wave's rows has kept so far
  // (uniform), and the size of this workgroup's region of a row's buffer
  uint32_t fcnt[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) fcnt[rr] = 0;
  const uint32_t fsub = FILT ? (uint32_t)(a.cap / stride) : 0u;

  auto run = [&](auto role_tag) {
    constexpr WaveRole role = decltype(role_tag)::value;
    // The rows of a wave are taken in groups of G (one or two): a unit of
    // work is one 32-key half of a page for one group. Lanes < 32 end up
    // with the group's first row, lanes >= 32 with its second.
    constexpr int G = RPW < 2 ? RPW : 2;
    constexpr int NG = RPW / G;
    // One row per wave: each half page leaves a partial head sum per lane
    // (16 heads); the two halves are completed together by one lane-half
    // swap, after which lane l holds the score of key l of the page. The
    // additions are the same, in the same order, as for a half at a time.
    auto head_sum = [&](const f32x16& acc) {
      float sum = 0.f;
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) sum = __builtin_fmaf(wv[i2], relu(acc[i2]), sum);
      return sum;
    };
    auto finish_page = [&](float p0, float p1, float ksl, int i) {
      if (i < 0) return;
      const float v = halves_sum_pair(p0, p1) * ksl;
      if constexpr (FILT) {
        if (wr0 >= nr) return;  // the wave's row is past the group's last (uniform)
        const int page_pos = (jx + i * stride) * kBlock;
        const int pos = page_pos + lane;
        // the keys of the page the row sees: lanes below nv (all but on its last page)
        const int nv = pos0 + wr0 - page_pos + 1;
        const uint64_t vis = nv >= 64 ? ~0ull : (nv <= 0 ? 0ull : (1ull << nv) - 1);
        const uint64_t m = __ballot(v >= thr_w[0]) & vis;
        if (m) {
          const bool keep = v >= thr_w[0] && lane < nv;  // this lane's bit of m
          const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          const uint32_t slot = fcnt[0] + rank;
          if (keep && slot < fsub)
            a.cand[(row0 + wr0) * (size_t)a.cap + (size_t)jx * fsub + slot] = make_uint2(ordered_key(v), (uint32_t)pos);
          fcnt[0] += (uint32_t)__popcll(m);
        }
      } else {
        sc_s[i % (LAG + 1)][wr0][lane] = v;
      }
    };
    // head-weighted ReLU sum of one unit (keys 32h .. 32h+31 of the i-th
    // page, rows gi*G ..) into the LDS score buffer
    auto epilogue = [&](const f32x16(&acc)[G], float ks, int i, int h, int gi) {
      float p[G];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        float sum = 0.f;
        if constexpr (RPW == 1) {
#pragma unroll
          for (int i2 = 0; i2 < 16; ++i2) sum = __builtin_fmaf(wv[i2], relu(acc[r][i2]), sum);
        } else {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(&w_s[wr0 + gi * G + r][8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sum = __builtin_fmaf(w4[e], relu(acc[r][4 * q4 + e]), sum);
          }
        }
        p[r] = sum;
      }
      const float v = halves_sum_pair(p[0], p[G - 1]) * ks;
      // both lane halves write; with one row per group they write the same value
      const int rr = gi * G + (G == 2 ? g : 0);
      if constexpr (FILT) {
        // filtered decode: keep (key, position) of a score that reaches its
        // row's threshold in this workgroup's region of the row's buffer (a
        // few per page at long contexts); with one row per group only the
        // lower lane half keeps
        if (i >= 0) {
          const int half_pos = (jx + i * stride) * kBlock + 32 * h;  // the half's first key
          const int pos = half_pos + n;
          // keys of the half each row sees (uniform): the group's first row
          // in lanes < 32, its second above; a row past the group's last
          // sees none, and so does the upper half with one row per group
          const int nva = wr0 + gi * G < nr ? pos0 + wr0 + gi * G - half_pos + 1 : 0;
          const int nvb = G == 2 && wr0 + gi * G + 1 < nr ? pos0 + wr0 + gi * G + 1 - half_pos + 1 : 0;
          auto lanes_below = [](int nv) { return nv >= 32 ? ~0u : (nv <= 0 ? 0u : (1u << nv) - 1u); };
          const uint64_t vis = (uint64_t)lanes_below(nva) | ((uint64_t)lanes_below(nvb) << 32);
          // the two thresholds are read as values, then selected per lane half:
          // a select of their addresses would put the arrays in scratch
          float thr_a = thr_w[gi * G], thr_b = thr_w[gi * G + G - 1];
          asm volatile("" : "+v"(thr_a), "+v"(thr_b));
          const float thr_rr = (G == 2 && g) ? thr_b : thr_a;
          const uint64_t m = __ballot(v >= thr_rr) & vis;
          if (m) {
            const bool keep = v >= thr_rr && n < (g ? nvb : nva);  // this lane's bit of m
            const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
            const uint32_t rank = g == 0 ? __builtin_amdgcn_mbcnt_lo(mlo, 0u) : __builtin_amdgcn_mbcnt_hi(mhi, 0u);
            uint32_t f_a = fcnt[gi * G], f_b = fcnt[gi * G + G - 1];
            asm volatile("" : "+v"(f_a), "+v"(f_b));
            const uint32_t slot = (g == 0 ? f_a : f_b) + rank;
            if (keep && slot < fsub)
              a.cand[(row0 + wr0 + rr) * (size_t)a.cap + (size_t)jx * fsub + slot] =
                  make_uint2(ordered_key(v), (uint32_t)pos);
            fcnt[gi * G] += (uint32_t)__popc(mlo);
            if constexpr (G == 2) fcnt[gi * G + 1] += (uint32_t)__popc(mhi);
          }
        }
      } else {
        if (i >= 0) sc_s[i % (LAG + 1)][wr0 + rr][32 * h + n] = v;
      }
    };
    // wave 3: store the group's scores of page i (complete once barrier i + LAG passed);
    // in the filtered decode, keep the (key, position) of each score >= its
    // row's threshold in this workgroup's region instead (rare: a few per
    // page at long contexts)
    auto flush = [&](int i) {
      if constexpr (FILT) {
        (void)i;  // filtered decode: the waves kept their candidates themselves
      } else {
        const uint32_t off = 4u * (uint32_t)((jx + i * stride) * kBlock + lane);
#pragma unroll
        for (int gr = 0; gr < ROWS; ++gr)  // descriptors rebuilt here: scalar work, no registers held
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc_s[i % (LAG + 1)][gr][lane]), row_rsrc(gr), off, 0,
                                                0);
      }
    };
    // FP8 keys pass both scale operands as 0: the compiler then emits the
    // plain v_mfma_f32_32x32x64_f8f6f4 (no scaling), which overlaps better
    // with VALU work than the scaled opcode (4% faster prefill scoring, same
    // results). MXFP4 keys need the scaled opcode for their block scales.
    auto mfma_unit = [&](f32x16(&acc)[G], const i32x8(&Bh)[2], const int (&sb)[2], int gi) {
#pragma unroll
      for (int r = 0; r < G; ++r) {
        acc[r] = f32x16{};
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            acc[r] = KF4 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[gi * G + r][t][s], Bh[s], acc[r], 0, 4,
                                                                          0, 127, 0, sb[s])
                         : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[gi * G + r][t][s], Bh[s], acc[r], 0, 0,
                                                                          0, 0, 0, 0);
      }
    };
    // B operands of keys 32h .. 32h+31 of a staged page. MXFP4: lane half
    // g, step s reads the 16-byte chunk 2g + s of its key (one MX block) and
    // that block's E8M0 scale (sb).
    auto load_b = [&](const uint8_t* kbuf, const float* ksb, int h, i32x8(&Bh)[2], int (&sb)[2]) {
      const int key = 32 * h + n;
      if constexpr (KF4) {
        const uint32_t sw = __float_as_uint(ksb[key]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(kbuf + key * (kIdxDim / 2) +
                                                          (((2 * g + s) ^ ((key >> 2) & 3)) << 4));
          Bh[s] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
          sb[s] = (int)((sw >> (8 * (2 * g + s))) & 0xffu);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const u32x4 lo4 = *reinterpret_cast<const u32x4*>(kbuf + key_chunk_off(key, 4 * g + 2 * s));
          const u32x4 hi4 = *reinterpret_cast<const u32x4*>(kbuf + key_chunk_off(key, 4 * g + 2 * s + 1));
          Bh[s] = i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                        (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
          sb[s] = 127;
        }
      }
    };
    // kRing - 1 pages are in flight. A copier's only vector-memory
    // operations in the loop are its copies, so its vmcnt counts exactly
    // its copies of the pages after page i.
    auto wait_page = [&](int i) {
      if constexpr (role == kCopier) {
        if (i + kRing - 2 < n_my) {
          if constexpr (KF4) {
            if (wave < 2) wait_vmcnt<2 * (kRing - 2)>();
            else wait_vmcnt<kRing - 2>();
          } else {
            wait_vmcnt<kCopiesPerWave * (kRing - 2)>();
          }
        } else {
          wait_vmcnt<0>();
        }
      }
    };

    // Software pipeline over units: the MFMAs of one unit run while the
    // VALU epilogue of the unit before it (of this page or, for the first
    // unit, the last unit of the previous page) is issued between them.
    f32x16 acc[2][G];
#pragma unroll
    for (int r = 0; r < G; ++r) acc[1][r] = f32x16{};
    float ks_prev = 0.f;
    float p_half0 = 0.f;  // one row per wave: the current page's first-half partial sums
    for (int i = 0; i < n_my; ++i) {
      if ((i & 7) == 0) set_progress_priority(i, n_my);
      wait_page(i);
      lds_barrier();  // page i is in LDS; the slot of page i - 1 is free
      if constexpr (role == kCopier) {
        if (i + kRing - 1 < n_my) issue(i + kRing - 1);
      }
      if constexpr (role == kFlusher) {
        if (i >= LAG) flush(i - LAG);
      }
      const uint8_t* kbuf = key_s[i % kRing];
      const float* ksb = ks_s[i % kRing];
      // keys of both halves up front for one group per half; with two
      // groups the second half's keys are read when its first unit starts
      i32x8 B[NG == 1 ? 2 : 1][2];
      int SB[NG == 1 ? 2 : 1][2];
      load_b(kbuf, ksb, 0, B[0], SB[0]);
      if constexpr (NG == 1) load_b(kbuf, ksb, 1, B[NG == 1 ? 1 : 0], SB[NG == 1 ? 1 : 0]);
      // MXFP4 keys carry their scales inside the dot products (E8M0 per block)
      const float ks[2] = {KF4 ? 1.f : ksb[n], KF4 ? 1.f : ksb[32 + n]};
      const float ksl = KF4 ? 1.f : ksb[lane];  // one row per wave: the scale of key `lane`
#pragma unroll
      for (int u = 0; u < 2 * NG; ++u) {  // unit u: half u / NG, group u % NG
        const int h = u / NG, gi = u % NG;
        if constexpr (NG > 1) {
          if (u == NG) load_b(kbuf, ksb, 1, B[0], SB[0]);
        }
        mfma_unit(acc[u & 1], B[NG == 1 ? h : 0], SB[NG == 1 ? h : 0], gi);
        if constexpr (G == 1) {
          if (u == 0) finish_page(p_half0, head_sum(acc[1][0]), ks_prev, i - 1);  // the previous page
          else p_half0 = head_sum(acc[0][0]);
        } else {
          if (u == 0) epilogue(acc[1], ks_prev, i - 1, 1, NG - 1);  // last unit of the previous page
          else epilogue(acc[(u - 1) & 1], ks[(u - 1) / NG], i, (u - 1) / NG, (u - 1) % NG);
        }
      }
      ks_prev = G == 1 ? ksl : ks[1];
    }
    if constexpr (G == 1) finish_page(p_half0, head_sum(acc[1][0]), ks_prev, n_my - 1);
    else epilogue(acc[1], ks_prev, n_my - 1, 1, NG - 1);
    __syncthreads();  // the last scores are in LDS
    if constexpr (role == kFlusher) {
      for (int i = max(0, n_my - LAG); i < n_my; ++i) flush(i);
    }
    if constexpr (FILT) {  // this workgroup's true count per row (also past its region)
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr)
        if (wr0 + rr < nr && lane == 0) a.cand_count[(row0 + wr0 + rr) * kMaxFilterWg + jx] = fcnt[rr];
    }
  };
  if (wave < kCopiers) run(std::integral_constant<WaveRole, kCopier>{});
  else run(std::integral_constant<WaveRole, kFlusher>{});
}

// Workgroups of a variant that fit one CU at once (registers, LDS), from
// the runtime's occupancy calculator; computed once per variant.
template <int RPW, bool QFP8, bool KF4, bool FILT>
static int resident_per_cu() {
  static const int n = [] {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, score_kernel<RPW, QFP8, KF4, FILT>, kThreads, 0) !=
            hipSuccess ||
        v < 1)
      v = 1;
    return v;
  }();
  return n;
}

static int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups per row group: one round of resident workgroups over the whole
// grid, at least one per request, none past max_wg_pages pages and about two
// pages each at least. A single request gets all G (max_blk / G pages each);
// with several, request b gets 1 + floor(spare p_b / P) or more of them,
// spare = G - B, P = the pages of all requests <= B max_blk, so each walks
// fewer than P / spare + 1 pages.
template <int RPW, bool QFP8, bool KF4, bool FILT>
static long long grid_x(int B, int R, int max_ctx) {
  constexpr long long kMax = max_wg_pages<RPW>();
  const int groups = (R + 4 * RPW - 1) / (4 * RPW);
  const long long max_blk = (max_ctx + kBlock - 1) / kBlock;
  const long long slots = (long long)resident_per_cu<RPW, QFP8, KF4, FILT>() * cu_count();
  long long G = slots / groups;
  const long long most = (long long)B * ((max_blk + 1) / 2);
  if (G > most) G = most;
  const long long least = B == 1 ? (max_blk + kMax - 1) / kMax : (long long)B + ((long long)B * max_blk + kMax - 1) / kMax;
  if (G < least) G = least;
  if (G < B) G = B;
  return G;
}

template <int RPW, bool QFP8, bool KF4, bool FILT>
static void launch_variant(const ScoreArgs& a, int B, int max_ctx, hipStream_t st) {
  const int groups = (a.R + 4 * RPW - 1) / (4 * RPW);
  const long long G = grid_x<RPW, QFP8, KF4, FILT>(B, a.R, max_ctx);
  hipLaunchKernelGGL((score_kernel<RPW, QFP8, KF4, FILT>), dim3((unsigned)G, 1, groups), dim3(kThreads), 0, st, a,
                     B);
}

template <bool KF4>
static void launch_format(const ScoreArgs& a, int B, int max_ctx, bool q_fp8, hipStream_t st) {
  // Rows per wave: one for decode-sized requests; more when a request brings
  // many FP8 query rows (prefill chunks), so that more rows share each page.
  if (a.cand) {  // filtered decode
    if (q_fp8) {  // up to 16 E4M3 query rows per workgroup, as for stored scores
      if (a.R > 16) launch_variant<4, true, KF4, true>(a, B, max_ctx, st);
      else if (a.R > 4) launch_variant<2, true, KF4, true>(a, B, max_ctx, st);
      else launch_variant<1, true, KF4, true>(a, B, max_ctx, st);
    } else {
      if (a.R > 4) launch_variant<2, false, KF4, true>(a, B, max_ctx, st);
      else launch_variant<1, false, KF4, true>(a, B, max_ctx, st);
    }
  } else if (q_fp8) {
    if (a.R > 16) launch_variant<4, true, KF4, false>(a, B, max_ctx, st);
    else if (a.R > 4) launch_variant<2, true, KF4, false>(a, B, max_ctx, st);
    else launch_variant<1, true, KF4, false>(a, B, max_ctx, st);
  } else {
    // up to 8 verification rows read each page once
    if (a.R > 4) launch_variant<2, false, KF4, false>(a, B, max_ctx, st);
    else launch_variant<1, false, KF4, false>(a, B, max_ctx, st);
  }
}

hipError_t launch_index_score(const ScoreArgs& a, int B, int max_ctx, bool q_fp8, hipStream_t st) {
  if (a.key_fp4) launch_format<true>(a, B, max_ctx, q_fp8, st);
  else launch_format<false>(a, B, max_ctx, q_fp8, st);
  return hipGetLastError();
}


template <bool KF4, bool QFP8>
static int filter_grid_fmt(int B, int R, int max_ctx) {
  if constexpr (QFP8) {  // (bf16 rows never take the 16-row variant)
    if (R > 16) return (int)grid_x<4, QFP8, KF4, true>(B, R, max_ctx);
  }
  return (int)(R > 4 ? grid_x<2, QFP8, KF4, true>(B, R, max_ctx) : grid_x<1, QFP8, KF4, true>(B, R, max_ctx));
}

int filter_grid(int B, int R, int max_ctx, bool mxfp4, bool q_fp8) {
  if (q_fp8) return mxfp4 ? filter_grid_fmt<true, true>(B, R, max_ctx) : filter_grid_fmt<false, true>(B, R, max_ctx);
  return mxfp4 ? filter_grid_fmt<true, false>(B, R, max_ctx) : filter_grid_fmt<false, false>(B, R, max_ctx);
}

}  // namespace dsa
