// Lightning-indexer scoring on gfx950 MFMA.
//
// score(row, s) = sum_h w[row][h] * ReLU(q[row][h] . key_s) * key_scale[s]
// ("vLLM Day-0 Support for Kimi K3.1 Pro", section "What Kimi K3.1 Pro
// changes": 32 heads x 128 dims over one 132-byte FP8 key per token).
//
// Work decomposition. One wave owns up to 4 query rows of one request and
// streams 32-key tiles of that request's pages: every key byte is loaded from
// HBM once and used for all of the request's verification rows ("TokenSpeed
// Kimi K3.1", section "Reducing indexer overhead on AMD MI350X": each key is
// loaded once for all rows). The rows' query fragments stay in VGPRs for the
// whole scan. Per tile and row, the 32 heads x 32 keys dot products are one
// accumulator of v_mfma_f32_32x32x16_bf16 (bf16 queries; E4M3 keys widened to
// bf16 exactly) or v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 queries, raw E4M3
// keys). The 32x32 output layout puts 16 heads of one key in each lane, so the
// head-weighted ReLU reduction is 16 in-lane max+fma steps plus one
// permlane32 swap between the two lane halves.
//
// The K dimension (the 128 key dims) is permuted identically for both MFMA
// operands: lane half g owns dims [64g, 64g+64) of its key, loaded as four
// contiguous 16-byte reads, and K-step s of the bf16 MFMA uses dims
// 64g + 8s + [0,8) (of the FP8 MFMA: 64g + 32s + [0,32)).
//
// Key scales (and E4M3 query scales) are positive, so they factor out of the
// ReLU and are applied once per (row, key) after the head reduction.
#include "common.h"
#include "kernels.h"

namespace dsa {

template <int RPW, bool QFP8, bool HIST>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a, int blk_stride) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;   // lane half
  const int n = lane & 31;   // key within the tile (B/D column), head within the A tile
  const int b = blockIdx.y;
  const int R = a.R;
  const int r0 = blockIdx.z * RPW;
  const int nr = min(RPW, R - r0);
  const int L = a.ctx_len[b];
  const int pos0 = L - R + r0;            // position of the group's first row
  const int blk_lim = ((pos0 + nr - 1) >> 6) + 1;  // pages any row of the group sees
  const size_t row0 = (size_t)b * R + r0;

  __shared__ uint32_t lhist[HIST ? RPW * kHistBins : 1];
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < RPW * kHistBins; i += 256) lhist[i] = 0;
    __syncthreads();
  }

  const int first_blk = blockIdx.x * 4 + wave;
  if (first_blk < blk_lim) {
    // ---- query fragments and head weights, resident for the whole scan
    constexpr int KSTEPS = QFP8 ? 2 : 8;
    typedef typename std::conditional<QFP8, i32x8, bf16x8>::type AFrag;
    AFrag A[RPW][KSTEPS];
    float wv[RPW][16];
    float qs[RPW];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const size_t row = row0 + min(rr, nr - 1);
      if constexpr (QFP8) {
        const i32x8* qp = reinterpret_cast<const i32x8*>(
            reinterpret_cast<const uint8_t*>(a.q) + (row * kIdxHeads + n) * kIdxDim + 64 * g);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) A[rr][s] = qp[s];
        qs[rr] = a.q_scale[row];
      } else {
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            reinterpret_cast<const __bf16*>(a.q) + (row * kIdxHeads + n) * kIdxDim + 64 * g);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) A[rr][s] = qp[s];
        qs[rr] = 1.0f;
      }
      const uint16_t* wp = a.w + row * kIdxHeads;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int head = 8 * (i >> 2) + 4 * g + (i & 3);
        wv[rr][i] = __uint_as_float((uint32_t)wp[head] << 16);
      }
    }

    const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
    // ---- stream this wave's pages: blocks first_blk, first_blk + stride, ...
    int blk = first_blk;
    int page = table[blk];
    for (; blk < blk_lim; blk += blk_stride) {
      const int nblk = blk + blk_stride;
      const int next_page = nblk < blk_lim ? table[nblk] : 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int slot = 32 * h + n;
        const size_t tok = (size_t)page * kBlock + slot;
        const u32x4* kp = reinterpret_cast<const u32x4*>(a.key_fp8 + tok * kIdxDim + 64 * g);
        const u32x4 k0 = kp[0], k1 = kp[1], k2 = kp[2], k3 = kp[3];
        const float ks = a.key_scale[tok];
        const uint32_t kw[16] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3],
                                 k2[0], k2[1], k2[2], k2[3], k3[0], k3[1], k3[2], k3[3]};
        float p[RPW];
        if constexpr (QFP8) {
          i32x8 B0, B1;
#pragma unroll
          for (int i = 0; i < 8; ++i) { B0[i] = (int)kw[i]; B1[i] = (int)kw[8 + i]; }
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) {
            f32x16 acc = {};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[rr][0], B0, acc, 0, 0, 0, 127, 0, 127);
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[rr][1], B1, acc, 0, 0, 0, 127, 0, 127);
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) t = __builtin_fmaf(wv[rr][i], fmaxf(acc[i], 0.f), t);
            p[rr] = t;
          }
        } else {
          bf16x8 Bf[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) Bf[s] = e4m3x8_bf16(kw[2 * s], kw[2 * s + 1]);
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) {
            f32x16 acc = {};
#pragma unroll
            for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[rr][s], Bf[s], acc, 0, 0, 0);
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) t = __builtin_fmaf(wv[rr][i], fmaxf(acc[i], 0.f), t);
            p[rr] = t;
          }
        }
        // ---- combine the two lane halves; lanes <32 hold row j, lanes >=32 row j+HALF
        constexpr int HALF = (RPW + 1) / 2;
        const int tokpos = blk * kBlock + slot;
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
          const float tot = halves_sum_pair(p[j], (j + HALF < RPW) ? p[j + HALF] : 0.f);
          const int rr = j + g * HALF;
          if (rr < nr && tokpos <= pos0 + rr) {
            const float v = tot * ks * qs[rr < RPW ? rr : 0];
            a.scores[(row0 + rr) * a.ld + tokpos] = v;
            if constexpr (HIST) atomicAdd(&lhist[rr * kHistBins + (ordered_key(v) >> 21)], 1u);
          }
        }
      }
      page = next_page;
    }
  }

  if constexpr (HIST) {
    __syncthreads();
    for (int i = threadIdx.x; i < RPW * kHistBins; i += 256) {
      const uint32_t c = lhist[i];
      const int rr = i / kHistBins;
      if (c != 0 && rr < nr) atomicAdd(&a.hist[(row0 + rr) * kHistBins + (i % kHistBins)], c);
    }
  }
}

template <int RPW, bool QFP8>
static void launch_rpw(const ScoreArgs& a, dim3 grid, int stride, hipStream_t st) {
  if (a.hist)
    hipLaunchKernelGGL((score_kernel<RPW, QFP8, true>), grid, dim3(256), 0, st, a, stride);
  else
    hipLaunchKernelGGL((score_kernel<RPW, QFP8, false>), grid, dim3(256), 0, st, a, stride);
}

hipError_t launch_index_score(const ScoreArgs& a, int B, int max_ctx, bool q_fp8, hipStream_t st) {
  const int rpw = a.R < 4 ? a.R : 4;
  const int groups = (a.R + rpw - 1) / rpw;
  const int max_blk = (max_ctx + kBlock - 1) / kBlock;
  // About two waves per SIMD over the whole GPU; each wave then walks
  // ceil(pages / waves-per-group) pages of its request.
  const long long total = (long long)B * groups * max_blk;
  long long per_wave = (total + 2047) / 2048;
  if (per_wave < 1) per_wave = 1;
  int wgs = (int)((max_blk + 4 * per_wave - 1) / (4 * per_wave));
  if (wgs < 1) wgs = 1;
  const dim3 grid(wgs, B, groups);
  const int stride = wgs * 4;
  switch (rpw) {
    case 1: q_fp8 ? launch_rpw<1, true>(a, grid, stride, st) : launch_rpw<1, false>(a, grid, stride, st); break;
    case 2: q_fp8 ? launch_rpw<2, true>(a, grid, stride, st) : launch_rpw<2, false>(a, grid, stride, st); break;
    case 3: q_fp8 ? launch_rpw<3, true>(a, grid, stride, st) : launch_rpw<3, false>(a, grid, stride, st); break;
    default: q_fp8 ? launch_rpw<4, true>(a, grid, stride, st) : launch_rpw<4, false>(a, grid, stride, st); break;
  }
  return hipGetLastError();
}

}  // namespace dsa
