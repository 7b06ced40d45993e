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
// rows). The next page is in flight in registers while the current one is
// computed.
//
// The dot products run on v_mfma_scale_f32_32x32x64_f8f6f4 with the raw E4M3
// key bytes as the B operand (no conversion). Queries enter as E4M3:
//  * E4M3 queries (prefill chunks) are used as they are, their row scale
//    applied after the head reduction;
//  * bf16 queries are split exactly into two E4M3 terms, q * 2^e = hi + lo,
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
// permlane32 swap between the lane halves. 2^-e, the key scale and the
// query row scale are positive and are applied after the ReLU.
//
// K (the 128 key dims) is permuted identically in both operands: lane half
// g of a 32x32x64 step s holds dims 64g + 32s + [0, 32).
#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int kKeyBytes = kBlock * kIdxDim;  // one page of keys, 8 KB

// LDS position of 16-byte chunk j of key n within a staged page: rows of
// 128 B with the chunk index XOR-swizzled by (n >> 1) & 7 so that the 16
// lanes of each read phase hit distinct banks.
DSA_DEV int key_chunk_off(int n, int j) { return n * kIdxDim + ((j ^ ((n >> 1) & 7)) << 4); }

DSA_DEV uint32_t e4m3x2_from_f32(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

template <int RPW, bool QFP8, bool HIST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void score_kernel(ScoreArgs a) {
  constexpr int ROWS = 4 * RPW;
  constexpr int NT = QFP8 ? 1 : 2;  // E4M3 terms per query value
  __shared__ __attribute__((aligned(16))) uint8_t key_s[kKeyBytes];
  __shared__ float ks_s[kBlock];
  __shared__ __attribute__((aligned(16))) float w_s[ROWS][kIdxHeads];
  __shared__ uint32_t lhist[HIST ? ROWS * kHistBins : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;   // lane half
  const int n = lane & 31;   // A row (head) / B and D column (key)
  const int b = blockIdx.y;
  const int R = a.R;
  const int r0 = blockIdx.z * ROWS;           // first row of the group within the request
  const int nr = min(ROWS, R - r0);           // rows of the group that exist
  const int L = a.ctx_len[b];
  const int pos0 = L - R + r0;                // position of the group's first row
  const int blk_lim = ((pos0 + nr - 1) >> 6) + 1;  // pages any row of the group sees
  const size_t row0 = (size_t)b * R + r0;
  const int wr0 = wave * RPW;                 // this wave's first row within the group

  if constexpr (HIST) {
    for (int i = tid; i < ROWS * kHistBins; i += 256) lhist[i] = 0;
  }

  // ---- query fragments (E4M3 terms) and per-head weights for this wave's rows
  i32x8 A[RPW][NT][2];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int gr = min(wr0 + rr, nr - 1);  // clamp: rows past the group reuse a valid row, never written
    const size_t row = row0 + gr;
    float head_scale = 1.0f;  // multiplies the dot product of head n
    if constexpr (QFP8) {
      const i32x8* qp = reinterpret_cast<const i32x8*>(reinterpret_cast<const uint8_t*>(a.q) +
                                                       (row * kIdxHeads + n) * kIdxDim + 64 * g);
      A[rr][0][0] = qp[0];
      A[rr][0][1] = qp[1];
      head_scale = a.q_scale[row];
    } else {
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.q) +
                                                         (row * kIdxHeads + n) * kIdxDim + 64 * g);
      float x[64];
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 v = qp[c];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[8 * c + e] = (float)v[e];
          amax = fmaxf(amax, fabsf(x[8 * c + e]));
        }
      }
      amax = fmaxf(amax, __shfl_xor(amax, 32));  // whole head: both lane halves
      int ex = 0;
      if (amax > 0.f) {
        int e2;
        const float m = frexpf(amax, &e2);  // amax = m * 2^e2, m in [0.5, 1)
        ex = (m <= 0.875f ? 9 : 8) - e2;    // amax * 2^ex in (224, 448]
      }
      head_scale = ldexpf(1.0f, -ex);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          uint32_t hw = 0, lw = 0;
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float x0 = ldexpf(x[32 * s + 4 * d + e], ex), x1 = ldexpf(x[32 * s + 4 * d + e + 1], ex);
            const uint32_t hb = e4m3x2_from_f32(x0, x1);
            const auto hf = __builtin_amdgcn_cvt_pk_f32_fp8(hb, false);
            const uint32_t lb = e4m3x2_from_f32(x0 - hf[0], x1 - hf[1]);
            hw |= hb << (8 * e);
            lw |= lb << (8 * e);
          }
          A[rr][0][s][d] = (int)hw;
          A[rr][1][s][d] = (int)lw;
        }
      }
    }
    // head weights with the head's scale folded in: w_s[row][head]
    if (g == 0) {
      const float wv = __uint_as_float((uint32_t)a.w[row * kIdxHeads + n] << 16);
      w_s[wr0 + rr][n] = wv * head_scale;
    }
  }
  __syncthreads();
  // the 16 heads this lane reduces (rows 8*(i/4) + 4g + i%4 of the 32x32 tile);
  // kept in VGPRs for up to two rows per wave, read from LDS otherwise
  constexpr int WREG = RPW <= 2 ? RPW : 1;
  float wv[WREG][16];
#pragma unroll
  for (int rr = 0; rr < WREG; ++rr)
#pragma unroll
    for (int i = 0; i < 16; ++i) wv[rr][i] = w_s[wr0 + rr][8 * (i >> 2) + 4 * g + (i & 3)];

  // ---- stream pages: this workgroup takes blocks blockIdx.x, +gridDim.x, ...
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
  const int stride = gridDim.x;
  u32x4 st0, st1;  // 32 bytes of the next page per thread
  float sst = 0.f;
  auto fetch = [&](int blk) {
    const size_t page = (size_t)table[blk];
    const u32x4* src = reinterpret_cast<const u32x4*>(a.key_fp8 + page * kKeyBytes);
    st0 = src[tid];
    st1 = src[tid + 256];
    if (tid < kBlock) sst = a.key_scale[page * kBlock + tid];
  };
  int blk = blockIdx.x;
  if (blk < blk_lim) fetch(blk);
  for (; blk < blk_lim; blk += stride) {
    __syncthreads();  // the previous page is consumed
    {
      const int c0 = tid, c1 = tid + 256;  // chunk c: key c >> 3, chunk c & 7
      *reinterpret_cast<u32x4*>(key_s + key_chunk_off(c0 >> 3, c0 & 7)) = st0;
      *reinterpret_cast<u32x4*>(key_s + key_chunk_off(c1 >> 3, c1 & 7)) = st1;
      if (tid < kBlock) ks_s[tid] = sst;
    }
    if (blk + stride < blk_lim) fetch(blk + stride);
    __syncthreads();

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = 32 * h + n;
      i32x8 B[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 lo4 = *reinterpret_cast<const u32x4*>(key_s + key_chunk_off(key, 4 * g + 2 * s));
        const u32x4 hi4 = *reinterpret_cast<const u32x4*>(key_s + key_chunk_off(key, 4 * g + 2 * s + 1));
        B[s] = i32x8{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                     (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
      }
      const float ks = ks_s[key];
      float p[RPW];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) {
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[rr][t][s], B[s], acc, 0, 0, 0, 127, 0, 127);
        float sum = 0.f;
        if constexpr (RPW <= 2) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sum = __builtin_fmaf(wv[rr][i], fmaxf(acc[i], 0.f), sum);
        } else {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(&w_s[wr0 + rr][8 * q4 + 4 * g]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sum = __builtin_fmaf(w4[e], fmaxf(acc[4 * q4 + e], 0.f), sum);
          }
        }
        p[rr] = sum;
      }
      // combine lane halves: lanes < 32 get row j, lanes >= 32 row j + HALF
      constexpr int HALF = (RPW + 1) / 2;
      const int tokpos = blk * kBlock + key;
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const float tot = halves_sum_pair(p[j], (j + HALF < RPW) ? p[j + HALF] : p[j]);
        const int rr = (RPW == 1) ? 0 : j + g * HALF;
        if ((RPW == 1 && g == 1) || rr >= RPW) continue;
        const int gr = wr0 + rr;
        if (gr < nr && tokpos <= pos0 + gr) {
          const float v = tot * ks;
          a.scores[(row0 + gr) * a.ld + tokpos] = v;
          if constexpr (HIST) atomicAdd(&lhist[gr * kHistBins + (ordered_key(v) >> 21)], 1u);
        }
      }
    }
  }

  if constexpr (HIST) {
    __syncthreads();
    for (int i = tid; i < ROWS * kHistBins; i += 256) {
      const uint32_t c = lhist[i];
      const int gr = i / kHistBins;
      if (c != 0 && gr < nr) atomicAdd(&a.hist[(row0 + gr) * kHistBins + (i % kHistBins)], c);
    }
  }
}

template <int RPW, bool QFP8>
static void launch_variant(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (RPW <= 2) {
    if (a.hist) {
      hipLaunchKernelGGL((score_kernel<RPW, QFP8, true>), grid, dim3(256), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((score_kernel<RPW, QFP8, false>), grid, dim3(256), 0, st, a);
}

hipError_t launch_index_score(const ScoreArgs& a, int B, int max_ctx, bool q_fp8, hipStream_t st) {
  // Rows per wave: one for decode-sized requests; more when a request brings
  // many rows (prefill chunks), so that more rows share each staged page.
  int rpw = 1;
  if (a.R > 4) rpw = 2;
  if (q_fp8 && a.R > 16) rpw = 4;
  if (a.hist && rpw > 2) rpw = 2;
  const int groups = (a.R + 4 * rpw - 1) / (4 * rpw);
  const int max_blk = (max_ctx + kBlock - 1) / kBlock;
  // About three workgroups per CU over the whole grid, at least 2 pages each.
  long long per_req = (768 + (long long)B * groups - 1) / ((long long)B * groups);
  long long cap = (max_blk + 1) / 2;
  if (per_req > cap) per_req = cap;
  if (per_req < 1) per_req = 1;
  const dim3 grid((unsigned)per_req, B, groups);
  if (q_fp8) {
    switch (rpw) {
      case 1: launch_variant<1, true>(a, grid, st); break;
      case 2: launch_variant<2, true>(a, grid, st); break;
      default: launch_variant<4, true>(a, grid, st); break;
    }
  } else {
    if (rpw == 1) launch_variant<1, false>(a, grid, st);
    else launch_variant<2, false>(a, grid, st);
  }
  return hipGetLastError();
}

}  // namespace dsa
