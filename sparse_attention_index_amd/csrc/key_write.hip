// Index-key write: LayerNorm, E4M3 quantisation with one absmax scale, and
// the paged write of each new token's key.
//
// "TokenSpeed Kimi K3.1", section "Integrating sparse attention with the K3
// stack", step 1: one fused kernel normalises the new token's index key,
// quantises it to FP8 with a single scale and writes it into the cache (and
// the loader accepts LayerNorm as the only key normalisation).
//
// One wave per new token: lane l holds dims 2l and 2l + 1 of the 128.
//  1. mean and biased variance over the 128 dims (fp32, DPP wave sums);
//  2. y = (x - mean) / sqrt(var + eps) * weight + bias;
//  3. scale = max |y| / 448 (1 for an all-zero row), codes = E4M3(y / scale)
//     by the hardware conversion (round to nearest even), with y / scale
//     clamped to +-448 first (a quotient one rounding past 448 must not
//     become NaN);
//  4. the 2 codes of each lane go out as one 16-bit store into the token's
//     cache slot block_table[b][pos / 64] * 64 + pos % 64, and lane 0 stores
//     the scale. Rows whose position or page is out of range are skipped.
// The work is bandwidth-bound: 256 B read and 132 B written per token.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int kRowsPerWg = 4;  // one wave per row

// Sum over the wave, returned in every lane: rotations inside rows of 16
// (DPP), then the four row totals read back.
DSA_DEV float wave_sum_f32(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false));  // row_ror 1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false));  // row_ror 2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));  // row_ror 4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));  // row_ror 8
  return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
}

DSA_DEV float wave_max_f32(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48))));
}

__global__ __launch_bounds__(64 * kRowsPerWg) void index_key_write_kernel(KeyWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerWg + (threadIdx.x >> 6);
  if (row >= a.rows) return;  // whole waves
  const int b = row / a.R;
  const int pos = a.ctx_len[b] - a.R + row % a.R;
  if (pos < 0 || (pos >> 6) >= a.max_blocks) return;
  const int blk = a.block_table[(size_t)b * a.max_blocks + (pos >> 6)];
  if (blk < 0 || blk >= a.num_blocks) return;
  const size_t slot = (size_t)blk * kBlock + (pos & 63);

  const uint32_t kv = reinterpret_cast<const uint32_t*>(a.k)[(size_t)row * (kIdxDim / 2) + lane];  // 2 bf16
  const float x0 = __uint_as_float(kv << 16), x1 = __uint_as_float(kv & 0xffff0000u);
  const float mean = wave_sum_f32(x0 + x1) * (1.0f / kIdxDim);
  const float d0 = x0 - mean, d1 = x1 - mean;
  const float var = wave_sum_f32(d0 * d0 + d1 * d1) * (1.0f / kIdxDim);
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const float2 wt = reinterpret_cast<const float2*>(a.ln_weight)[lane];
  const float2 bs = reinterpret_cast<const float2*>(a.ln_bias)[lane];
  const float y0 = d0 * rstd * wt.x + bs.x, y1 = d1 * rstd * wt.y + bs.y;
  const float amax = wave_max_f32(fmaxf(fabsf(y0), fabsf(y1)));
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  const float v0 = fminf(fmaxf(y0 / scale, -448.0f), 448.0f);
  const float v1 = fminf(fmaxf(y1 / scale, -448.0f), 448.0f);
  const uint32_t codes = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false) & 0xffffu;
  reinterpret_cast<uint16_t*>(a.key_fp8 + slot * kIdxDim)[lane] = (uint16_t)codes;
  if (lane == 0) a.key_scale[slot] = scale;
}

hipError_t launch_index_key_write(const KeyWriteArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((a.rows + kRowsPerWg - 1) / kRowsPerWg);
  hipLaunchKernelGGL(index_key_write_kernel, dim3(grid), dim3(64 * kRowsPerWg), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
