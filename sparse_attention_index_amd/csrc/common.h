// Shared device types and helpers for the gfx950 DSA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define DSA_DEV __device__ __forceinline__

namespace dsa {

constexpr int kBlock = 64;      // tokens per cache page
constexpr int kIdxHeads = 32;   // indexer heads
constexpr int kIdxDim = 128;    // indexer head dim (bytes per FP8 key)
constexpr int kLat = 576;       // latent width
constexpr int kV = 512;         // value width
constexpr int kMlaHeads = 16;   // MLA heads per call
constexpr int kMaxTopk = 2048;
constexpr int kHistBins = 2048; // first radix digit: top 11 bits of the ordered key

// Four OCP E4M3 codes packed in a dword -> two bf16 pairs (exact).
DSA_DEV bf16x2 e4m3x2_lo_bf16(uint32_t w) { return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false); }
DSA_DEV bf16x2 e4m3x2_hi_bf16(uint32_t w) { return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true); }

// Eight E4M3 codes (two dwords) -> bf16x8 MFMA operand, element i = byte i.
DSA_DEV bf16x8 e4m3x8_bf16(uint32_t w0, uint32_t w1) {
  bf16x2 a = e4m3x2_lo_bf16(w0), b = e4m3x2_hi_bf16(w0), c = e4m3x2_lo_bf16(w1), d = e4m3x2_hi_bf16(w1);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// fp32 -> uint32 key whose unsigned order is the float order; -0 maps like +0.
DSA_DEV uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

DSA_DEV float bf16_to_f32(__bf16 x) { return (float)x; }

// Sum over the two 32-lane halves: returns (lanes 0-31: a_lo + a_hi, lanes 32-63: b_lo + b_hi).
DSA_DEV float halves_sum_pair(float a, float b) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// 16 (4) bytes per lane from global memory straight into LDS at
// lds_base + 16 (4) * lane; lds_base must be the same for the whole wave.
// Issued through inline asm so that the compiler neither counts these copies
// nor inserts waits for them: every consumer waits with wait_vmcnt below.
// M0 is set right before each copy; no compiler-generated instruction in the
// kernels using these relies on M0 (LDS accesses on gfx950 do not read it).
DSA_DEV void copy16_to_lds(const void* src, void* lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base) : "memory");
}
DSA_DEV void copy4_to_lds(const void* src, void* lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(base) : "memory");
}
// The same copies from a wave-uniform base plus a per-lane 32-bit byte
// offset (the base lives in scalar registers: no 64-bit address per lane).
DSA_DEV void copy16_to_lds_at(const void* sbase, uint32_t off, void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sbase), "s"(m0) : "memory");
}
DSA_DEV void copy4_to_lds_at(const void* sbase, uint32_t off, void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(sbase), "s"(m0) : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
DSA_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global->LDS copies.
DSA_DEV void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace dsa
