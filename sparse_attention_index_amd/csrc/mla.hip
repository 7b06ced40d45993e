// Sparse MLA over the selected latent rows, on gfx950 MFMA.
//
// "vLLM Day-0 Support for Kimi K3.1 Pro", section "What Kimi K3.1 Pro
// changes": MLA runs exactly over only the selected tokens. Each token's
// latent row is 576 FP8 values (512 compressed KV + 64 RoPE dims, "Kimi K3.1
// Pro on AMD Instinct", model overview) with one fp32 scale; the logits use
// all 576 dims and the values are the first 512.
//
// One workgroup (4 waves) handles one query row (16 heads) over a range of
// its selected positions, in tiles of 64 positions:
//  1. the 64 latent rows are gathered through the block table into LDS
//     (16-byte loads, one padded row per token);
//  2. QK: wave w computes the 16 heads x 16 tokens [16w, 16w+16) logits with
//     18 v_mfma_f32_16x16x32_bf16 steps (queries bf16 in VGPRs for the whole
//     call, latent E4M3 widened to bf16 exactly);
//  3. online softmax: running max and sum per head, combined across the 4
//     waves through LDS so that every wave rescales identically;
//  4. PV: probabilities (times the token's latent scale) go to LDS as bf16;
//     wave w accumulates out dims [128w, 128w+128) with 16x16x32 bf16 MFMA.
//     The V operand needs 8 consecutive tokens of one dim per lane; it comes
//     from the row-major LDS tile through ds_read_b64_tr_b8, which transposes
//     an 8x16 byte block across each 16-lane group.
// When a row's positions are split over several workgroups, each writes its
// unnormalised partial (out, max, sum) and a combine kernel merges them by
// log-sum-exp (the same algebra the pages use to merge decode-context-parallel
// partial outputs, "TokenSpeed Kimi K3.1", section "Sharding long contexts").
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int TK = 64;       // tokens per tile
static constexpr int PITCH = 592;   // LDS bytes per staged latent row (576 + 16 pad)
static constexpr int PP = 72;       // LDS bf16 per probability row (64 + 8 pad)
static constexpr int kChunks = kLat / 16;  // 16-byte chunks per latent row

struct MlaPart {
  float* o;   // [rows][splits][16][512]
  float* ml;  // [rows][splits][16][2]  (max, sum)
  int splits;
  int keys_per_split;
};

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

DSA_DEV i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void sparse_mla_kernel(MlaArgs a, MlaPart part) {
  __shared__ __attribute__((aligned(16))) uint8_t lat_s[TK * PITCH];
  __shared__ __attribute__((aligned(16))) __bf16 p_s[kMlaHeads * PP];
  __shared__ int32_t rowaddr_s[kMaxTopk];
  __shared__ float scl_s[TK];
  __shared__ float red_s[2][4][kMlaHeads];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;   // 16-lane group
  const int n = lane & 15;
  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int b = row / a.R;
  const int kbeg = split * part.keys_per_split;
  const int kend = min(a.k, kbeg + part.keys_per_split);
  const int nkeys = max(0, kend - kbeg);
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
  const int32_t* sel = a.idx + (size_t)row * a.k;

  // Resolve every selected position of this split to a cache row up front
  // (-1: skipped), so the tile loop has no dependent index loads.
  for (int j = tid; j < nkeys; j += 256) {
    int32_t ra = -1;
    const int pos = sel[kbeg + j];
    if (pos >= 0 && pos < a.max_blocks * kBlock) ra = table[pos >> 6] * kBlock + (pos & 63);
    rowaddr_s[j] = ra;
  }

  // Query fragments: lane holds head n, dims 32s + 8g + [0,8) for step s.
  bf16x8 qa[18];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.q) +
                                                       ((size_t)row * kMlaHeads + n) * kLat + 8 * g);
#pragma unroll
    for (int s = 0; s < 18; ++s) qa[s] = qp[4 * s];
  }

  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
  __syncthreads();

  // Each thread moves 9 of the tile's 64 x 36 sixteen-byte chunks; the next
  // tile's chunks are in flight while the current one is computed.
  constexpr int kPer = TK * kChunks / 256;
  u32x4 stage[kPer];
  float sstage = 0.f;
  auto load_tile = [&](int t0) {
    if (tid < TK) {
      const int ra = (t0 + tid < nkeys) ? rowaddr_s[t0 + tid] : -1;
      sstage = ra >= 0 ? a.lat_scale[ra] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + 256 * i;
      const int r = c / kChunks;
      const int q16 = c - r * kChunks;
      const int ra = (t0 + r < nkeys) ? rowaddr_s[t0 + r] : -1;
      stage[i] = u32x4{0u, 0u, 0u, 0u};
      if (ra >= 0) stage[i] = *reinterpret_cast<const u32x4*>(a.lat_fp8 + (size_t)ra * kLat + q16 * 16);
    }
  };
  if (nkeys > 0) load_tile(0);

  for (int t0 = 0; t0 < nkeys; t0 += TK) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + 256 * i;
      const int r = c / kChunks;
      const int q16 = c - r * kChunks;
      *reinterpret_cast<u32x4*>(lat_s + r * PITCH + q16 * 16) = stage[i];
    }
    if (tid < TK) scl_s[tid] = sstage;
    if (t0 + TK < nkeys) load_tile(t0 + TK);
    __syncthreads();

    // QK: logits for tokens 16*wave + n, heads 4g + i
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* kr = lat_s + (16 * wave + n) * PITCH + 8 * g;
#pragma unroll
      for (int s = 0; s < 18; ++s) {
        const uint2 v = *reinterpret_cast<const uint2*>(kr + 32 * s);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], e4m3x8_bf16(v.x, v.y), sacc, 0, 0, 0);
      }
    }
    const int tok = 16 * wave + n;
    const bool valid = (t0 + tok < nkeys) && rowaddr_s[t0 + tok] >= 0;
    const float sc = valid ? scl_s[tok] : 0.f;
    const float f = a.sm_scale * sc;
    float x[4], mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = valid ? sacc[i] * f : -INFINITY;
      mx[i] = x[i];
    }
    // online softmax: per-head max and sum over the tile's 64 tokens
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], off));
    if (n == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_s[0][wave][4 * g + i] = mx[i];
    __syncthreads();
    float alpha[4], p[4], sm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const float tmax = fmaxf(fmaxf(red_s[0][0][h], red_s[0][1][h]), fmaxf(red_s[0][2][h], red_s[0][3][h]));
      const float mnew = fmaxf(m_run[i], tmax);
      alpha[i] = (mnew == -INFINITY) ? 1.f : __expf(m_run[i] - mnew);
      p[i] = (x[i] == -INFINITY) ? 0.f : __expf(x[i] - mnew);
      m_run[i] = mnew;
      sm[i] = p[i];
      p_s[h * PP + tok] = (__bf16)(p[i] * sc);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm[i] += __shfl_xor(sm[i], off);
    if (n == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_s[1][wave][4 * g + i] = sm[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const float tsum = red_s[1][0][h] + red_s[1][1][h] + red_s[1][2][h] + red_s[1][3][h];
      l_run[i] = l_run[i] * alpha[i] + tsum;
    }

    // PV: out[:, 128w .. 128w+128) += P . V
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[j][i] *= alpha[i];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(p_s + n * PP + 32 * s + 8 * g);
      const uint8_t* vrow = lat_s + (32 * s + 8 * g + (n >> 1)) * PITCH + 128 * wave + 8 * (n & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const i32x2 v = lds_read_tr8(vrow + 16 * j);
        o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, e4m3x8_bf16((uint32_t)v[0], (uint32_t)v[1]), o[j], 0, 0,
                                                       0);
      }
    }
    __syncthreads();
  }

  // Output: lane holds dims 128w + 16j + n, heads 4g + i.
  if (part.splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const float inv = l_run[i] > 0.f ? 1.f / l_run[i] : 0.f;
      __bf16* orow = reinterpret_cast<__bf16*>(a.out) + ((size_t)row * kMlaHeads + h) * kV;
#pragma unroll
      for (int j = 0; j < 8; ++j) orow[128 * wave + 16 * j + n] = (__bf16)(o[j][i] * inv);
      if (a.lse && wave == 0 && n == 0)
        a.lse[(size_t)row * kMlaHeads + h] = l_run[i] > 0.f ? m_run[i] + __logf(l_run[i]) : -INFINITY;
    }
  } else {
    const size_t base = (size_t)row * part.splits + split;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      float* orow = part.o + (base * kMlaHeads + h) * kV;
#pragma unroll
      for (int j = 0; j < 8; ++j) orow[128 * wave + 16 * j + n] = o[j][i];
      if (wave == 0 && n == 0) {
        part.ml[(base * kMlaHeads + h) * 2 + 0] = m_run[i];
        part.ml[(base * kMlaHeads + h) * 2 + 1] = l_run[i];
      }
    }
  }
}

// Merge split partials: out = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}.
// Grid (8, rows): workgroup x handles dims [64x, 64x + 64) of all 16 heads.
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaPart part, uint16_t* out_bits, float* lse) {
  __shared__ float wgt_s[64][kMlaHeads];  // per split, per head weight e^{m_s - M} / L
  const int row = blockIdx.y;
  const int S = part.splits;
  const float* ml = part.ml + (size_t)row * S * kMlaHeads * 2;
  if (threadIdx.x < kMlaHeads) {
    const int h = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[(s * kMlaHeads + h) * 2]);
    float L = 0.f;
    for (int s = 0; s < S; ++s) {
      const float m = ml[(s * kMlaHeads + h) * 2];
      L += (m == -INFINITY) ? 0.f : ml[(s * kMlaHeads + h) * 2 + 1] * __expf(m - M);
    }
    for (int s = 0; s < S; ++s) {
      const float m = ml[(s * kMlaHeads + h) * 2];
      wgt_s[s][h] = (L > 0.f && m != -INFINITY) ? __expf(m - M) / L : 0.f;
    }
    if (lse && blockIdx.x == 0) lse[(size_t)row * kMlaHeads + h] = L > 0.f ? M + __logf(L) : -INFINITY;
  }
  __syncthreads();
  __bf16* out = reinterpret_cast<__bf16*>(out_bits) + (size_t)row * kMlaHeads * kV;
  const float* po = part.o + (size_t)row * S * kMlaHeads * kV;
  // 16 heads x 64 dims = 1024 outputs, 4 per thread (one float4 per split)
  const int h = threadIdx.x >> 4;
  const int d = 64 * blockIdx.x + 4 * (threadIdx.x & 15);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(po + ((size_t)s * kMlaHeads + h) * kV + d);
    const float wgt = wgt_s[s][h];
    acc += v * wgt;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) out[h * kV + d + e] = (__bf16)acc[e];
}

static int splits_for(int rows, int k) {
  int s = (512 + rows - 1) / rows;  // aim at ~512 workgroups
  const int max_s = (k + TK * 4 - 1) / (TK * 4);  // at least four tiles per split
  if (s > max_s) s = max_s;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

size_t mla_ws_bytes(int rows, int k, bool split) {
  if (!split) return 0;
  const int S = splits_for(rows, k);
  if (S == 1) return 0;
  return (size_t)rows * S * kMlaHeads * (kV + 2) * sizeof(float) + 256;
}

hipError_t launch_sparse_mla(const MlaArgs& a, int rows, bool split, void* ws, hipStream_t st) {
  MlaPart part;
  part.splits = split ? splits_for(rows, a.k) : 1;
  int kps = (a.k + part.splits - 1) / part.splits;
  kps = (kps + TK - 1) / TK * TK;

  part.keys_per_split = kps;
  part.o = reinterpret_cast<float*>(ws);
  part.ml = part.o ? part.o + (size_t)rows * part.splits * kMlaHeads * kV : nullptr;
  hipLaunchKernelGGL(sparse_mla_kernel, dim3(part.splits, rows), dim3(256), 0, st, a, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || part.splits == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(kV / 64, rows), dim3(256), 0, st, part, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
