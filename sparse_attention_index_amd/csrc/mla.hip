// Sparse MLA over the selected latent rows, on gfx950 MFMA.
//
// "vLLM Day-0 Support for Kimi K3.1 Pro", section "What Kimi K3.1 Pro
// changes": MLA runs exactly over only the selected tokens. Each token's
// latent row is 576 FP8 values (512 compressed KV + 64 RoPE dims, "Kimi K3.1
// Pro on AMD Instinct", model overview) with one fp32 scale; the logits use
// all 576 dims and the values are the first 512.
//
// One workgroup (8 waves, one workgroup per CU) handles one query row (16
// heads) over a range of its selected positions, in tiles of 128 positions:
//  1. gather: the tile's 128 latent rows (72 KB) are copied from HBM straight
//     into LDS with global_load_lds_dwordx4 (no VGPR staging) into a ring of
//     two tile buffers, so the next tile is in flight while one is computed.
//     Completion is tracked with explicit vmcnt waits and raw s_barrier (a
//     full __syncthreads would also wait for the copy in flight). Rows are
//     stored unpadded with their 16-byte chunks rotated by row / 4
//     (chunk_slot), which spreads both read patterns below over distinct
//     LDS banks;
//  2. QK: wave w computes the logits of 16 heads x 16 tokens [16w, 16w+16)
//     with FP8 MFMAs on the raw E4M3 latent (no conversion): the bf16 query
//     is split into two E4M3 terms (exact down to ~2^-10 of the head's
//     largest element) with a power-of-two block scale
//     per head, once per workgroup, and stays in VGPRs for the whole call;
//  3. online softmax against a per-head reference shared by all waves: p =
//     exp(logit - reference). The reference only moves when a logit of the
//     tile exceeds it by more than kSlack (always on the first tile with a
//     valid token); only then do the waves exchange tile maxima (DPP row
//     reductions, then LDS) and rescale the partial output and sums, so the
//     common tile needs one barrier for the softmax instead of two. Row sums
//     stay per lane and are combined once at the end;
//  4. PV: probabilities (times the token's latent scale) go to LDS as bf16;
//     wave w accumulates out dims [64w, 64w+64) with 16x16x32 bf16 MFMA.
//     The V operand needs 8 consecutive tokens of one dim per lane; it comes
//     from the row-major LDS tile through ds_read_b64_tr_b8, which transposes
//     an 8x16 byte block across each 16-lane group.
// When a row's positions are split over several workgroups, each writes its
// unnormalised partial (out, max, sum) and a combine kernel merges them by
// log-sum-exp (the same algebra the pages use to merge decode-context-parallel
// partial outputs, "TokenSpeed Kimi K3.1", section "Sharding long contexts").
#include <math.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

namespace dsa {

static constexpr int TK = 128;                        // tokens per tile
static constexpr int NBUF = 2;                       // tile buffers in the LDS ring
static constexpr int kChunks = kLat / 16;            // 16-byte chunks per latent row
static constexpr int TILE_B = TK * kLat;             // 73,728 bytes
static constexpr int kWaves = 8;
static constexpr int kPer = TK * kChunks / (64 * kWaves);  // chunk copies per lane per tile (9)
static constexpr int PP = TK + 8;                    // LDS bf16 per probability row (padded)
static constexpr float kSlack = 8.f;                 // p stays below e^8 against a lagging reference

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

// Where chunk j of tile row r sits within the row: rotated by r / 4, the
// 32 chunks of the 512 value dims among themselves and the 4 chunks of the
// 64 RoPE dims among themselves. A row is 144 dwords, 16 banks on from the
// one before, so 16 consecutive rows (an aligned block) reading the same
// chunk land on 16 distinct groups of 4 banks: (4 (r mod 4) + r / 4 + j)
// mod 16 differs for every r of the block. Both tile reads below take such
// blocks (16 rows per 16-lane group of 16-byte reads, 16 rows per 32 lanes
// of 8-byte transposed reads).
DSA_DEV int chunk_slot(int r, int j) {
  const int q = r >> 2;
  return j < 32 ? (j + q) & 31 : 32 + ((j + q) & 3);
}
// The chunk held by slot s of row r (the inverse).
DSA_DEV int slot_chunk(int r, int s) {
  const int q = r >> 2;
  return s < 32 ? (s - q) & 31 : 32 + ((s - 32 - q) & 3);
}
// LDS byte offset of 16-byte chunk j of tile row r.
DSA_DEV int lat_off(int r, int j) { return r * kLat + chunk_slot(r, j) * 16; }

// Max / sum over the 16 lanes of a DPP row (row_ror 1, 2, 4, 8).
template <int CTRL>
DSA_DEV float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
DSA_DEV float row_max16(float v) {
  v = fmaxf(v, dpp_f<0x121>(v));
  v = fmaxf(v, dpp_f<0x122>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  return fmaxf(v, dpp_f<0x128>(v));
}
DSA_DEV float row_sum16(float v) {
  v += dpp_f<0x121>(v);
  v += dpp_f<0x122>(v);
  v += dpp_f<0x124>(v);
  return v + dpp_f<0x128>(v);
}

__global__ __launch_bounds__(512) void sparse_mla_kernel(MlaArgs a, MlaPart part) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[NBUF][TILE_B];
  __shared__ __attribute__((aligned(16))) float scl_r[NBUF][TK];
  __shared__ __attribute__((aligned(16))) __bf16 p_s[kMlaHeads * PP];
  __shared__ float mx_s[kWaves][kMlaHeads];
  __shared__ __attribute__((aligned(8))) uint8_t flag_s[kWaves];  // per wave: a logit passed the reference
  __shared__ int32_t rowaddr_s[kMaxTopk];
  __shared__ uint32_t tile_bad[kMaxTopk / TK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;   // 16-lane group
  const int n = lane & 15;
  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int qrow = a.q_rows ? row % a.q_rows : row;  // the query row (and request) this row attends for
  const int b = qrow / a.R;
  const int kbeg = split * part.keys_per_split;
  const int kend = min(a.nvalid ? a.nvalid[row] : a.k, min(a.k, kbeg + part.keys_per_split));
  const int nkeys = max(0, kend - kbeg);
  const int ntiles = (nkeys + TK - 1) / TK;
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
  const int32_t* sel = a.idx + (size_t)row * a.k;

  // Resolve every selected position of this split to a cache row up front
  // (-1: skipped; also the padding of the last tile).
  if (a.slots) {  // the selection arrives as cache rows already
    const int32_t* sl = a.slots + (size_t)row * a.k;
    for (int j = tid; j < ntiles * TK; j += 512) rowaddr_s[j] = j < nkeys ? sl[kbeg + j] : -1;
  } else {
    for (int j = tid; j < ntiles * TK; j += 512) {
      int32_t ra = -1;
      if (j < nkeys) {
        const int pos = sel[kbeg + j];
        if (pos >= 0 && pos < a.max_blocks * kBlock) ra = table[pos >> 6] * kBlock + (pos & 63);
      }
      rowaddr_s[j] = ra;
    }
  }
  // This thread's share of the query for the split below: head tid / 32,
  // dims 18 (tid % 32) + [0, 18), as 9 pairs of bf16.
  uint32_t qpair[9];
  {
    const uint32_t* qp = reinterpret_cast<const uint32_t*>(a.q) +
                         (((size_t)qrow * kMlaHeads + (tid >> 5)) * kLat + 18 * (tid & 31)) / 2;
#pragma unroll
    for (int j = 0; j < 9; ++j) qpair[j] = qp[j];
  }
  __syncthreads();  // rowaddr_s complete
  if (tid < ntiles) {
    uint32_t bad = 0;
    for (int r = 0; r < TK; ++r) bad |= (uint32_t)(rowaddr_s[tid * TK + r] < 0);
    tile_bad[tid] = bad;
  }

  // This lane's copy map, the same for every tile: chunk slot
  // c_i = 64 (9 wave + i) + lane of the tile holds row r_i, global chunk j_i.
  int cr[kPer], cj[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = 64 * (kPer * wave + i) + lane;
    cr[i] = c / kChunks;
    cj[i] = slot_chunk(cr[i], c - cr[i] * kChunks);
  }
  // Copy tile t into ring slot t % 2 (skipped rows read row 0 and are zeroed
  // after arrival). Waves 0 and 1 also copy the tile's 128 scales.
  // Copies i0 .. i1-1 of this wave for tile t; the part ending at kPer also
  // takes the scales. A tile's copies go out in three parts spread over the
  // previous tile's compute: a wave issuing many gathers at once stalls on
  // the full memory queue while the others wait for it at the next barrier.
  auto issue = [&](int t, int i0, int i1) {
    uint8_t* dst = ring[t % NBUF];
    const int rb = t * TK;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (i < i0 || i >= i1) continue;
      const int ra = rowaddr_s[rb + cr[i]];
      const uint8_t* src = a.lat_fp8 + (size_t)(ra >= 0 ? ra : 0) * kLat + cj[i] * 16;
      copy16_to_lds(src, dst + 1024 * (kPer * wave + i));
    }
    if (i1 == kPer && wave < 2) {
      const int ra = rowaddr_s[rb + 64 * wave + lane];
      copy4_to_lds(a.lat_scale + (ra >= 0 ? ra : 0), &scl_r[t % NBUF][64 * wave]);
    }
  };

  f32x4 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run: the softmax reference of each head, the same in every wave; it is
  // the running maximum except that it only moves when a logit exceeds it by
  // more than kSlack (then p <= e^kSlack). l_run: this lane's partial sum of
  // p over the tokens it held, relative to m_run.
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
  wait_vmcnt<0>();  // nothing but the copies is outstanding from here on
  if (ntiles > 0) issue(0, 0, kPer);

  // Query as the A operand of 16x16x128 FP8 MFMAs. Each bf16 value is split
  // exactly into two E4M3 terms, q 2^e = hi + lo, with a power of two 2^e
  // per head that puts the head's largest magnitude in (224, 448]; 2^-e goes
  // back in through the MFMA's A-operand block scale. (bf16 carries 8
  // significant bits, each E4M3 term 4; only elements ~2^10 below the head
  // maximum lose low bits, to E4M3's subnormal step.) The workgroup splits
  // the query once, each thread 18 values, into [head][656] byte planes
  // staged in ring slot 1 (dims 576-639 zero), which tile 1's copies only
  // overwrite after the loop's first barrier; lane (g, n) then reads head
  // n, dims 128s + 32g + [0, 32) of step s.
  i32x8 qh[5], ql[5];
  int qscale;  // E8M0 exponent of 2^-e for this lane's head
  {
    constexpr int kQRow = 656;  // 640 bytes per head plus 16: the 16 heads' rows start on distinct banks
    uint8_t* qhi = ring[1];
    uint8_t* qlo = ring[1] + kMlaHeads * kQRow;
    int* ex_s = reinterpret_cast<int*>(ring[1] + 2 * kMlaHeads * kQRow);
    const int hq = tid >> 5, kq = tid & 31;
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 9; ++j)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(qpair[j] << 16)), fabsf(__uint_as_float(qpair[j] & 0xffff0000u))));
    amax = row_max16(amax);
    amax = fmaxf(amax, __shfl_xor(amax, 16));  // the 32 threads of a head
    int ex = 0;
    if (amax > 0.f) {
      int e2;
      const float fr = frexpf(amax, &e2);  // amax = fr 2^e2, fr in [0.5, 1)
      ex = max(min((fr <= 0.875f ? 9 : 8) - e2, 127), -127);
    }
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      const float x0 = ldexpf(__uint_as_float(qpair[j] << 16), ex);
      const float x1 = ldexpf(__uint_as_float(qpair[j] & 0xffff0000u), ex);
      const uint32_t hb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false) & 0xffffu;
      const auto hf = __builtin_amdgcn_cvt_pk_f32_fp8(hb, false);
      const uint32_t lb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0 - hf[0], x1 - hf[1], 0, false) & 0xffffu;
      *reinterpret_cast<uint16_t*>(qhi + hq * kQRow + 18 * kq + 2 * j) = (uint16_t)hb;
      *reinterpret_cast<uint16_t*>(qlo + hq * kQRow + 18 * kq + 2 * j) = (uint16_t)lb;
    }
    if (kq < 16) {
      *reinterpret_cast<uint32_t*>(qhi + hq * kQRow + kLat + 4 * kq) = 0u;
      *reinterpret_cast<uint32_t*>(qlo + hq * kQRow + kLat + 4 * kq) = 0u;
    }
    if (kq == 0) ex_s[hq] = ex;
    lds_barrier();  // staged (the tile-0 copies stay in flight)
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      const u32x4* ph = reinterpret_cast<const u32x4*>(qhi + n * kQRow + 128 * s + 32 * g);
      const u32x4* pl = reinterpret_cast<const u32x4*>(qlo + n * kQRow + 128 * s + 32 * g);
      const u32x4 h0 = ph[0], h1 = ph[1], l0 = pl[0], l1 = pl[1];
      qh[s] = i32x8{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
      ql[s] = i32x8{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
    }
    qscale = 127 - ex_s[n];
  }

  for (int t = 0; t < ntiles; ++t) {
    uint8_t* tile = ring[t % NBUF];
    float* scl = scl_r[t % NBUF];
    wait_vmcnt<0>();  // tile t is the only copy in flight
    if (tile_bad[t]) {  // zero the skipped rows this lane copied
      const int rb = t * TK;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (rowaddr_s[rb + cr[i]] < 0)
          *reinterpret_cast<u32x4*>(tile + 16 * (64 * (kPer * wave + i) + lane)) = u32x4{0u, 0u, 0u, 0u};
      if (wave < 2 && rowaddr_s[rb + 64 * wave + lane] < 0) scl[64 * wave + lane] = 0.f;
    }
    lds_barrier();  // tile t complete in LDS for all waves; tile t-1 fully consumed
    const bool more = t + 1 < ntiles;  // tile t + 1 goes into the slot tile t - 1 used
    if (more) issue(t + 1, 0, 3);

    // QK: logits for tokens 16*wave + n, heads 4g + i (D layout); lane
    // (g, n) supplies token n's dims 128s + 32g + [0, 32) as the B operand,
    // two 16-byte chunks of its row with no conversion (step 4, groups 2-3:
    // a repeat of valid chunks, multiplied by zero queries)
    const int tok = 16 * wave + n;
    f32x4 sacc;
    {
      f32x4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
      int tk = tok;
      asm volatile("" : "+v"(tk));  // offsets recomputed per tile rather than held in registers
      const uint8_t* kr = tile + tk * kLat;
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        int c = 8 * s + 2 * g;  // even: c and c + 1 are both value or both RoPE chunks
        if (c >= kChunks) c -= 4;
        const u32x4 lo4 = *reinterpret_cast<const u32x4*>(kr + 16 * chunk_slot(tk, c));
        const u32x4 hi4 = *reinterpret_cast<const u32x4*>(kr + 16 * chunk_slot(tk, c + 1));
        const i32x8 bk = {(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                          (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        ah = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qh[s], bk, ah, 0, 0, 0, qscale, 0, 127);
        al = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ql[s], bk, al, 0, 0, 0, qscale, 0, 127);
      }
      sacc = ah + al;
    }
    if (more) issue(t + 1, 3, 6);
    // Softmax against the current reference. Only if some logit of the tile
    // exceeds it by more than kSlack (always on the first tile with a valid
    // token) do the waves exchange tile maxima and move the reference, which
    // rescales the partial output and sums; the result is the same either way.
    const bool valid = rowaddr_s[t * TK + tok] >= 0;
    const float sc = scl[tok];
    const float f = a.sm_scale * sc;
    float x[4], p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = valid ? sacc[i] * f : -INFINITY;
    // The first tile always sets the reference (it starts at -inf), so it
    // goes straight to the exchange of tile maxima.
    bool exchange = true;
    if (t > 0) {
      bool over = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        over |= x[i] > m_run[i] + kSlack;
        p[i] = (x[i] == -INFINITY) ? 0.f : __expf(x[i] - m_run[i]);
        p_s[(4 * g + i) * PP + tok] = (__bf16)(p[i] * sc);
      }
      const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;  // all lanes take part
      if (lane == 0) flag_s[wave] = wave_over ? 1 : 0;
      lds_barrier();
      exchange = *reinterpret_cast<const uint64_t*>(flag_s) != 0;
    }
    if (exchange) {  // every wave reads the same flags: a uniform branch
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float mx = row_max16(x[i]);
        if (n == 0) mx_s[wave][4 * g + i] = mx;
      }
      lds_barrier();
      float alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * g + i;
        float tmax = mx_s[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) tmax = fmaxf(tmax, mx_s[w][h]);
        const float mnew = fmaxf(m_run[i], tmax);
        alpha[i] = (mnew == -INFINITY) ? 1.f : __expf(m_run[i] - mnew);
        p[i] = (x[i] == -INFINITY) ? 0.f : __expf(x[i] - mnew);
        m_run[i] = mnew;
        p_s[h * PP + tok] = (__bf16)(p[i] * sc);
        l_run[i] *= alpha[i];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[j][i] *= alpha[i];
      lds_barrier();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) l_run[i] += p[i];
    if (more) issue(t + 1, 6, kPer);

    // PV: out[:, 64w .. 64w+64) += P . V over the tile's 128 tokens
#pragma unroll
    for (int s = 0; s < TK / 32; ++s) {
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(p_s + n * PP + 32 * s + 8 * g);
      const int r = 32 * s + 8 * g + (n >> 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i32x2 v = lds_read_tr8(tile + lat_off(r, 4 * wave + j) + 8 * (n & 1));
        o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, e4m3x8_bf16((uint32_t)v[0], (uint32_t)v[1]), o[j], 0, 0,
                                                       0);
      }
    }
  }

  // Row sums: every lane holds the part of its own tokens.
#pragma unroll
  for (int i = 0; i < 4; ++i) l_run[i] = row_sum16(l_run[i]);
  // mx_s is free: its last reads in the loop were followed by a barrier
  if (n == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx_s[wave][4 * g + i] = l_run[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l += mx_s[w][h];
    l_run[i] = l;
  }

  // Output: lane holds dims 64w + 16j + n, heads 4g + i.
  if (part.splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const float inv = l_run[i] > 0.f ? 1.f / l_run[i] : 0.f;
      __bf16* orow = reinterpret_cast<__bf16*>(a.out) + ((size_t)row * kMlaHeads + h) * kV;
#pragma unroll
      for (int j = 0; j < 4; ++j) orow[64 * wave + 16 * j + n] = (__bf16)(o[j][i] * inv);
      if (a.lse && wave == 0 && n == 0)
        a.lse[(size_t)row * kMlaHeads + h] = l_run[i] > 0.f ? m_run[i] + __logf(l_run[i]) : -INFINITY;
    }
  } else {
    // partials are read once, by the merge: streamed stores (nontemporal)
    const size_t base = (size_t)row * part.splits + split;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      float* orow = part.o + (base * kMlaHeads + h) * kV;
#pragma unroll
      for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(o[j][i], &orow[64 * wave + 16 * j + n]);
      if (wave == 0 && n == 0) {
        __builtin_nontemporal_store(m_run[i], &part.ml[(base * kMlaHeads + h) * 2 + 0]);
        __builtin_nontemporal_store(l_run[i], &part.ml[(base * kMlaHeads + h) * 2 + 1]);
      }
    }
  }
}

// Merge split partials: out = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}.
// Grid (8, rows): workgroup x handles dims [64x, 64x + 64) of all 16 heads;
// thread t owns head h = t / 16 and dims 64x + 4 (t % 16) + [0, 4). Every
// global load is issued up front (the first 8 splits' partial outputs, and
// the (max, sum) pairs of splits t % 16 + 16 u), so the merge costs one memory
// round trip; the 16 lanes of a head reduce with DPP.
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaPart part, uint16_t* out_bits, float* lse) {
  __shared__ float wgt_s[64][kMlaHeads];  // per split, per head weight e^{m_s - M} / L
  const int row = blockIdx.y;
  const int S = part.splits;  // <= 64
  const int h = threadIdx.x >> 4, j = threadIdx.x & 15;
  const int d = 64 * blockIdx.x + 4 * j;
  const float* po = part.o + (size_t)row * S * kMlaHeads * kV + h * kV + d;
  constexpr size_t kSplitStride = (size_t)kMlaHeads * kV;
  // The first 16 splits' partial outputs are loaded before the weights are
  // known, all at once: every load is issued (splits past the last re-read
  // it; those values are never used), no branch waits on one of them.
  constexpr int kFirst = 16;
  f32x4 v[kFirst];
#pragma unroll
  for (int u = 0; u < kFirst; ++u) v[u] = *reinterpret_cast<const f32x4*>(po + (u < S ? u : S - 1) * kSplitStride);
  const float2* ml = reinterpret_cast<const float2*>(part.ml) + (size_t)row * S * kMlaHeads;
  float m[4], l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int s = j + 16 * u;
    const float2 x = ml[(s < S ? s : S - 1) * kMlaHeads + h];
    m[u] = s < S ? x.x : -INFINITY;
    l[u] = s < S ? x.y : 0.f;
  }
  const float M = row_max16(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])));
  float L = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) L += m[u] == -INFINITY ? 0.f : l[u] * __expf(m[u] - M);
  L = row_sum16(L);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int s = j + 16 * u;
    if (s < S) wgt_s[s][h] = (L > 0.f && m[u] != -INFINITY) ? __expf(m[u] - M) / L : 0.f;
  }
  if (lse && blockIdx.x == 0 && j == 0) lse[(size_t)row * kMlaHeads + h] = L > 0.f ? M + __logf(L) : -INFINITY;
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kFirst; ++u)
    if (u < S) acc += v[u] * wgt_s[u][h];
  for (int s0 = kFirst; s0 < S; s0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = s0 + u < S ? *reinterpret_cast<const f32x4*>(po + (s0 + u) * kSplitStride) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) acc += v[u] * wgt_s[s0 + u][h];
  }
  __bf16* out = reinterpret_cast<__bf16*>(out_bits) + ((size_t)row * kMlaHeads + h) * kV + d;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = (__bf16)acc[e];
}

static int splits_for(int rows, int k) {
  int s = (256 + rows - 1) / rows;  // aim at one workgroup per CU
  const int max_s = (k + TK - 1) / TK;  // at least one tile per split
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
  hipLaunchKernelGGL(sparse_mla_kernel, dim3(part.splits, rows), dim3(512), 0, st, a, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || part.splits == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(kV / 64, rows), dim3(256), 0, st, part, a.out, a.lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------ no-allocation scratch

// The split partials of the no-allocation decode entry point live in this
// array of the library's own device memory (one copy per GPU, held until
// the process ends). 16 MiB is the most mla_ws_bytes asks for at any row
// count (255 rows in two splits of k = 2048: 255 * 2 * 16 * 514 * 4 + 256
// bytes); 256 rows and more take one split and no scratch.
static constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

size_t mla_scratch_bytes() { return kScratchBytes; }

// The device address of `scratch` on the current device, looked up once per
// device (the host-side name is a stand-in, not a device address).
hipError_t mla_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace dsa
