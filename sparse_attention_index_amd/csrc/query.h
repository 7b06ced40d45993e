// The indexer query as MFMA operands, shared by the scoring kernels: a bf16
// query row split into two E4M3 terms under one power-of-two scale per
// head, or E4M3 query codes as they are, in the K order the key operands
// use; and the ReLU of the head-weighted reduction.
#pragma once

#include "common.h"
#include "kernels.h"

namespace dsa {

// max(x, 0) as one integer max on the bit pattern: non-negative floats
// (+0 included) are non-negative integers, negative floats and -0 are
// negative integers. The operands are finite MFMA sums.
DSA_DEV float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

DSA_DEV uint32_t e4m3x2_from_f32(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}


// The E4M3 A operands of one query row: q * 2^e = hi + lo (bf16 queries) or
// the query codes as they are, with the factor 2^-e (or the row scale) that
// multiplies the head's dot products. fetch_query loads the lane's raw bytes;
// finish_query converts them, later, while the first key pages are in flight.
//
// K order. With FP8 keys, byte i of lane half g's operand for step s is dim
// 64g + 32s + i. With MXFP4 keys the FP4 B operand of lane half g holds K
// indices 16g + [0, 16) in its first 16 nibbles and 32 + 16g + [0, 16) in
// the next 16 (measured on gfx950), and its one E8M0 scale covers all 32;
// so that those 32 values are one MX block (dims 64g + 32s + [0, 32), read
// as 16 contiguous bytes), the query's byte i of lane half g, step s, must
// be dim 32s + 16g + i (i < 16) or 64 + 32s + 16g + i - 16 (i >= 16).
template <bool QFP8, bool KF4>
struct QueryRaw {
  u32x4 v[8];  // bf16 queries: 64 values per lane
};
template <bool KF4>
struct QueryRaw<true, KF4> {
  u32x4 p[4];  // E4M3 codes: 64 per lane
  float scale;
};

template <bool QFP8, bool KF4>
DSA_DEV void fetch_query(const ScoreArgs& a, size_t row, int n, int g, QueryRaw<QFP8, KF4>& r) {
  if constexpr (QFP8) {
    const uint8_t* q8 = reinterpret_cast<const uint8_t*>(a.q) + (row * kIdxHeads + n) * kIdxDim;
#pragma unroll
    for (int c = 0; c < 4; ++c)  // MXFP4 keys: dims 32c + 16g + [0, 16); FP8 keys: dims 64g + 16c + [0, 16)
      r.p[c] = *reinterpret_cast<const u32x4*>(q8 + (KF4 ? 32 * c + 16 * g : 64 * g + 16 * c));
    r.scale = a.q_scale[row];
  } else {
    const u32x4* qp = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(a.q) +
                                                     (row * kIdxHeads + n) * kIdxDim);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // piece c of 8 values: FP8 keys: dims 64g + 8c; MXFP4 keys: dims
      // 16g + 32u + 8(c & 1) for u = 0, 2, 1, 3 (c >> 1 = 0..3)
      const int u = (c >> 1) == 1 ? 2 : ((c >> 1) == 2 ? 1 : (c >> 1));
      r.v[c] = KF4 ? qp[(16 * g + 32 * u) / 8 + (c & 1)] : qp[8 * g + c];
    }
  }
}

// Keeps the code that reads r after this point of the program (the raw
// registers pass through an empty asm statement).
template <bool QFP8, bool KF4>
DSA_DEV void hold_query(QueryRaw<QFP8, KF4>& r) {
  if constexpr (QFP8) {
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(r.p[c]));
    asm volatile("" : "+v"(r.scale));
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(r.v[c]));
  }
}

template <bool QFP8, bool KF4>
DSA_DEV float finish_query(const QueryRaw<QFP8, KF4>& r, i32x8 (&A)[QFP8 ? 1 : 2][2]) {
  if constexpr (QFP8) {
    auto cat = [](const u32x4& x, const u32x4& y) {
      return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    };
    A[0][0] = KF4 ? cat(r.p[0], r.p[2]) : cat(r.p[0], r.p[1]);
    A[0][1] = KF4 ? cat(r.p[1], r.p[3]) : cat(r.p[2], r.p[3]);
    return r.scale;
  } else {
    // x[32s + i]: the value at byte i of step s
    float x[64];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, r.v[c]);
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
        A[0][s][d] = (int)hw;
        A[1][s][d] = (int)lw;
      }
    }
    return ldexpf(1.0f, -ex);
  }
}

}  // namespace dsa
