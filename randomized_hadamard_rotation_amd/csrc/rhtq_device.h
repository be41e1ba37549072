// Device helpers shared by the HIP kernels (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "rhtq.h"

namespace rhtq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Streaming accesses: each input and output byte is touched once, so the loads and
// stores carry the non-temporal hint (measured ~10% more HBM throughput on gfx950).
__device__ __forceinline__ uint4 ld_stream(const uint16_t* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
// fp32 input: four values as their bit patterns.
__device__ __forceinline__ uint4 ld_stream(const float* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
// fp32 values as three bf16 terms, packed in pairs for the MFMA A operand: hi keeps the top 16
// bits of each value (truncation); mid8 is the top 16 bits of what is left, times 2^8; lo16 the
// rest times 2^16, which has at most 8 significant bits and so is a bf16 exactly.  Every step is
// exact, so x = hi + 2^-8 mid8 + 2^-16 lo16.  The factors keep the lower terms about as large as
// the value itself: unscaled, they would be bf16 denormals for values below about 2^-110, and
// the matrix cores flush denormal operands (rows near 1e-37 lost 2^-8 of their precision).  Pair
// k holds elements 2k (low half) and 2k + 1 (high half).
__device__ __forceinline__ void split3_bf16(const uint4& r0, const uint4& r1, uint32_t (&hi)[4], uint32_t (&mid8)[4],
                                            uint32_t (&lo16)[4]) {
  const uint32_t e[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  uint32_t m[8], l[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float r8 = (__uint_as_float(e[k]) - __uint_as_float(e[k] & 0xFFFF0000u)) * 256.0f;
    m[k] = __float_as_uint(r8);
    l[k] = __float_as_uint((r8 - __uint_as_float(m[k] & 0xFFFF0000u)) * 256.0f);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    hi[k] = __builtin_amdgcn_perm(e[2 * k + 1], e[2 * k], 0x07060302u);
    mid8[k] = __builtin_amdgcn_perm(m[2 * k + 1], m[2 * k], 0x07060302u);
    lo16[k] = __builtin_amdgcn_perm(l[2 * k + 1], l[2 * k], 0x07060302u);
  }
}

// Term t (0, 1, 2) of the exact split of an fp32 value (bit pattern v) into three bf16 values
// v = hi + mid + lo, each returned as an fp32 bit pattern whose low 16 bits are zero: hi keeps the
// top 16 bits of v, mid the top 16 bits of v - hi, and lo = v - hi - mid has at most 8
// significant bits.  Unlike split3_bf16 the terms are not rescaled, so they can share one
// accumulator: below about 2^-110 the lower terms are bf16 denormals, which the matrix cores
// read as zero.
__device__ __forceinline__ uint32_t f32_term(uint32_t v, int t) {
  const uint32_t hi = v & 0xFFFF0000u;
  if (t == 0) return hi;
  const float r = __uint_as_float(v) - __uint_as_float(hi);
  const uint32_t mid = __float_as_uint(r) & 0xFFFF0000u;
  if (t == 1) return mid;
  return __float_as_uint(r - __uint_as_float(mid));
}

// Stage-1 products of fp32 input: the three terms through the same +-1 operand, each into its
// own accumulator (the scaled terms must not meet the hi products unscaled), then
// d = dh + 2^-8 dm + 2^-16 dl.
__device__ __forceinline__ f32x4 stage1_f32(const bf16x8& ah, const bf16x8& am, const bf16x8& al, const bf16x8& b) {
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4 dh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, z, 0, 0, 0);
  const f32x4 dm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b, z, 0, 0, 0);
  const f32x4 dl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, z, 0, 0, 0);
  f32x4 d;
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = __builtin_fmaf(dl[i], 1.0f / 65536.0f, __builtin_fmaf(dm[i], 1.0f / 256.0f, dh[i]));
  return d;
}

__device__ __forceinline__ void st_stream(uint8_t* p, uint32_t a, uint32_t b) {
  const u32x2 t = {a, b};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_stream(uint8_t* p, uint32_t a) {
  __builtin_nontemporal_store(a, reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void st_stream(float* p, float a, float b, float c, float d) {
  const f32x4 t = {a, b, c, d};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
}

// INT4 group scale from the group maximum of the unnormalised values:
// s = amax * cnorm * fl(1/7) stored as fp32 or fp16 (nearest even, saturating); inv maps an
// unnormalised value to scale units (0 for a zero group); clamp flags a stored scale far
// below amax / 7 (fp16 saturation, subnormal scale) where codes must be clamped to [-8, 7].
struct Int4Scale {
  float s;
  float inv;
  bool clamp;
};

__device__ __forceinline__ Int4Scale int4_scale(float amax, float cnorm, int scale_dtype) {
  Int4Scale r;
  r.s = (amax * cnorm) * (1.0f / 7.0f);   // within 2 ulp of the exact quotient
  const float sq = scale_dtype == RHTQ_SCALE_F32 ? r.s : __half2float(__float2half_rn(fminf(r.s, 65504.0f)));
  r.inv = sq > 0.0f ? cnorm * __builtin_amdgcn_rcpf(sq) : 0.0f;
  r.clamp = amax * r.inv > 7.25f;
  return r;
}

// Constant +-1 MFMA operands, per lane, as compile-time tables (one 16-byte load per lane
// instead of building them with popcounts at kernel start):
//  b1[t][lane]: B operand of v_mfma_f32_16x16x32_bf16 for a 32-point Sylvester Hadamard,
//    B_t[x][n] = H32[x][2n + t] with x = 8 (lane >> 4) + e and n = lane & 15, so output
//    column n of N-tile t is element 2n + t of the transformed 32-vector (bf16).
//  b16[t][lane]: as b1 for 16-wide rows, the block-diagonal I2 (x) H16: element bit 4 selects
//    the row, so B_t[x][n] = H16[x & 15][(2n + t) & 15] where x and 2n + t share bit 4, else 0.
//  s2[t2][lane]: stage-2 B operand of v_mfma_f32_16x16x32_f16, the H32 over element bits
//    5-9: k = 8 (lane >> 4) + e stands for bits 5,6 = e & 3, bits 7,8 = lane >> 4,
//    bit 9 = e >> 2; column n = lane & 15 stands for output bits 5-8 and tile t2 for
//    output bit 9 (f16).
struct alignas(16) H32Operands {
  uint16_t b1[2][64][8];
  uint16_t b16[2][64][8];
  uint16_t s2[2][64][8];
  uint16_t s2n[2][64][8];   // s2 negated
  constexpr H32Operands() : b1(), b16(), s2(), s2n() {
    for (int t = 0; t < 2; ++t)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          const int xk = 8 * (lane >> 4) + e, o = 2 * (lane & 15) + t;
          b1[t][lane][e] = (__builtin_popcount(xk & o) & 1) ? 0xBF80 : 0x3F80;
          b16[t][lane][e] = ((xk ^ o) & 16) ? 0x0000 : ((__builtin_popcount(xk & o & 15) & 1) ? 0xBF80 : 0x3F80);
          const int k = (e & 3) | ((lane >> 4) << 2) | ((e >> 2) << 4), n = (lane & 15) | (t << 4);
          s2[t][lane][e] = (__builtin_popcount(k & n) & 1) ? 0xBC00 : 0x3C00;
          s2n[t][lane][e] = (uint16_t)(s2[t][lane][e] ^ 0x8000);
        }
  }
};
// b1 and b16 as f16 (+-1 and 0 are exact in both): the B operands of v_mfma_f32_16x16x32_f16
// when the input itself is fp16.
struct alignas(16) H32OperandsF16 {
  uint16_t b1h[2][64][8];
  uint16_t b16h[2][64][8];
  constexpr H32OperandsF16() : b1h(), b16h() {
    const H32Operands h;
    for (int t = 0; t < 2; ++t)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          b1h[t][lane][e] = (uint16_t)((h.b1[t][lane][e] & 0x8000) | 0x3C00);
          b16h[t][lane][e] = h.b16[t][lane][e] ? (uint16_t)((h.b16[t][lane][e] & 0x8000) | 0x3C00) : (uint16_t)0;
        }
  }
};
namespace {
__constant__ H32Operands kH32Ops;
__constant__ H32OperandsF16 kH32OpsF16;
}

// The stage-1 operands as raw 16-bit patterns: bf16 +-1, or f16 +-1 for fp16 input (H16).
template <bool H16 = false>
__device__ __forceinline__ bf16x8 h32_operand(int lane, int t) {
  bf16x8 r;
  if constexpr (H16) __builtin_memcpy(&r, &kH32OpsF16.b1h[t][lane][0], 16);
  else __builtin_memcpy(&r, &kH32Ops.b1[t][lane][0], 16);
  return r;
}

template <bool H16 = false>
__device__ __forceinline__ bf16x8 h16_operand(int lane, int t) {
  bf16x8 r;
  if constexpr (H16) __builtin_memcpy(&r, &kH32OpsF16.b16h[t][lane][0], 16);
  else __builtin_memcpy(&r, &kH32Ops.b16[t][lane][0], 16);
  return r;
}

// One stage-1 product, c + A B with A eight input values per lane (sign bits already flipped)
// and B a +-1 operand from h32_operand / h16_operand of the same type: bf16 input on the bf16
// instruction, fp16 input (H16) on the f16 one.  Both read their operands exactly.
template <bool H16>
__device__ __forceinline__ f32x4 stage1_mma(bf16x8 av, bf16x8 hb, f32x4 c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, hb), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb, c, 0, 0, 0);
}


// (a, b) -> (a + b, a - b): one Walsh-Hadamard butterfly.
__device__ __forceinline__ void bfly(float& a, float& b) {
  const float s = a + b;
  b = a - b;
  a = s;
}

// Order-12 Williamson Hadamard array
//   [[ A,  B,  B,  B],
//    [-B,  A, -B,  B],
//    [-B,  B,  A, -B],
//    [-B, -B,  B,  A]]      A = J3 (all ones), B = J3 - 2 I3,
// entry (r, c) as +1 / -1.  Block (bi, bj) is negated when bit 4*bi + bj of 0x3950 is set.
__host__ __device__ constexpr int h12_entry(int r, int c) {
  const int bi = r / 3, bj = c / 3;
  const int bsign = ((0x3950 >> (4 * bi + bj)) & 1) ? -1 : 1;
  const int e = (bi == bj) ? 1 : ((r % 3) == (c % 3) ? -1 : 1);
  return bsign * e;
}

// Order-172 factor (QuaRot reviews, review 2 Questions: 172 is the non-power-of-two part of
// the Llama 2 7B width): the same Williamson array with four symmetric circulants A, B, C, D
// of order 43 in place of A, B, B, B, so block (bi, bj) holds circulant bi ^ bj, negated
// under the same mask 0x3950.  Circulant t has entry (r, c) = f_t((c - r) mod 43) with
// f_t(0) = +1 and, for k != 0, f_t(k) = -1 exactly when the coset of k modulo the order-6
// subgroup {1, 6, 7, 36, 37, 42} of the units mod 43 is in the mask kNeg43[t]; coset
// index = (discrete log of k to base 3) mod 7.  Then A^2 + B^2 + C^2 + D^2 = 172 I.
constexpr uint32_t kNeg43[4] = {0x70u, 0x59u, 0x45u, 0x13u};

// Coset index of every k in 1..42 ((discrete log of k to base 3) mod 7); entry 0 unused.
struct Coset43 {
  int8_t c[43];
  constexpr Coset43() : c() {
    int p = 1;
    for (int e = 0; e < 42; ++e) {
      c[p] = (int8_t)(e % 7);
      p = (p * 3) % 43;
    }
  }
};
constexpr Coset43 kCoset43{};

__host__ __device__ constexpr int h172_entry(int r, int c) {
  const int bi = r / 43, bj = c / 43;
  const int bsign = ((0x3950 >> (4 * bi + bj)) & 1) ? -1 : 1;
  const int k = ((c % 43) - (r % 43) + 43) % 43;
  const int e = (k == 0) ? 1 : (((kNeg43[bi ^ bj] >> kCoset43.c[k]) & 1) ? -1 : 1);
  return bsign * e;
}

// Bit j of word w[i][j >> 5] is set when H172[i][j] = -1 (T: of H172^T).
template <bool T>
struct H172Bits {
  uint32_t w[172][6];
  constexpr H172Bits() : w() {
    for (int i = 0; i < 172; ++i)
      for (int j = 0; j < 172; ++j)
        if ((T ? h172_entry(j, i) : h172_entry(i, j)) < 0) w[i][j >> 5] |= 1u << (j & 31);
  }
};

// w <- H12 w using the array's structure: with v1..v4 the four 3-blocks, sk = sum(vk),
// A v = sk * 1 and B v = sk * 1 - 2 v, so block k of the result is
// T_k * 1 + 2 (+-vi +-vj +-vl) with T_k = +-s1 +-s2 +-s3 +-s4 (52 adds/FMAs per 12 values).
__device__ __forceinline__ void h12_forward(float* w) {
  const float s1 = w[0] + w[1] + w[2];
  const float s2 = w[3] + w[4] + w[5];
  const float s3 = w[6] + w[7] + w[8];
  const float s4 = w[9] + w[10] + w[11];
  const float pa = s1 + s3, pb = s2 + s4, pc = s2 - s4, pd = s3 - s1;
  const float t1 = pa + pb, t2 = pb - pa, t3 = pc + pd, t4 = pd - pc;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const float v1 = w[k], v2 = w[3 + k], v3 = w[6 + k], v4 = w[9 + k];
    const float s34 = v3 + v4, d34 = v3 - v4, d24 = v2 - v4, s12 = v1 + v2;
    w[k] = __builtin_fmaf(-2.0f, v2 + s34, t1);       // -2 (v2 + v3 + v4)
    w[3 + k] = __builtin_fmaf(2.0f, v1 + d34, t2);    // +2 (v1 + v3 - v4)
    w[6 + k] = __builtin_fmaf(2.0f, v1 - d24, t3);    // +2 (v1 - v2 + v4)
    w[9 + k] = __builtin_fmaf(2.0f, s12 - v3, t4);    // +2 (v1 + v2 - v3)
  }
}

// Maximum of non-negative values over aligned groups of G lanes (G a power of two,
// 1..64); every lane of the group receives it.  Non-negative floats order like their
// bit patterns, so the comparisons are unsigned integer maxima, which fold the DPP lane
// moves into the max.  Within 16 lanes by DPP; across rows by the gfx950 lane swaps.
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ float group_max(float v, int G) {
  uint32_t u = __float_as_uint(v);
  if (G >= 2) u = umax(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));
  if (G >= 4) u = umax(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));
  if (G >= 8) u = umax(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false));
  if (G >= 16) u = umax(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false));
  if (G >= 32) {
    auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    u = umax(p[0], p[1]);
  }
  if (G >= 64) {
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    u = umax(p[0], p[1]);
  }
  return __uint_as_float(u);
}

// ---- two-stage matrix-core transform helpers ----

__device__ __forceinline__ f16x8 h32_stage2_operand(int lane, int t2) {
  f16x8 r;
  __builtin_memcpy(&r, &kH32Ops.s2[t2][lane][0], 16);
  return r;
}

// The stage-2 operand negated.
__device__ __forceinline__ f16x8 h32_stage2_operand_neg(int lane, int t2) {
  f16x8 r;
  __builtin_memcpy(&r, &kH32Ops.s2n[t2][lane][0], 16);
  return r;
}

// Maxima of non-negative values compare as unsigned bit patterns (see group_max).
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  const uint32_t u = __float_as_uint(v);
  return __uint_as_float(umax(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, CTRL, 0xF, 0xF, false)));
}

// Pairwise exchange across lane bit 4 (rows of 16 lanes 0<->1, 2<->3) followed by max:
// the result holds a's maxima in rows 0 and 2 and b's in rows 1 and 3.
__device__ __forceinline__ float swap16_max(float a, float b) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(umax(p[0], p[1]));
}
// Same across lane bit 5 (halves of 32 lanes): a's maxima in rows 0-1, b's in rows 2-3.
__device__ __forceinline__ float swap32_max(float a, float b) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(umax(p[0], p[1]));
}
// Inverse of the compaction: x holds (rows 0, 2 -> a; rows 1, 3 -> b); returns a and b
// broadcast over the row pairs.
__device__ __forceinline__ void expand16(float x, float& a, float& b) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(p[0]);
  b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void expand32(float x, float& a, float& b) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(p[0]);
  b = __uint_as_float(p[1]);
}

// Power-of-two split scale for a row whose largest |stage-1 value| has the bits mb:
// S = 2^(14 - e) with e the exponent of that maximum, so |y S| < 2^15; returned with
// its inverse, both kept within the normal range.
__device__ __forceinline__ void split_scale(uint32_t mb, float& S, float& invS) {
  int be = 268 - (int)((mb >> 23) & 0xFF);   // biased exponent of 2^(14 - e)
  be = be < 1 ? 1 : (be > 253 ? 253 : be);
  S = __uint_as_float((uint32_t)be << 23);
  invS = __uint_as_float((uint32_t)(254 - be) << 23);
}

// Eight values y scaled by S, split into f16 pairs: hi = f16(y S) and lo = f16(y S - hi),
// both nearest even; y S - hi is exact in fp32, so hi + lo carries 22 significant bits.
// Word k of hi / lo holds elements 2k (low half) and 2k + 1 (high half).  Written with
// v_fma_mixlo/mixhi_f16 so that each half costs one instruction and lo reads hi through
// op_sel; the order keeps every half-register write at least one instruction away from
// its reader, and the closing s_nop covers the VALU-write to matrix-core-read distance.
// The compiler places no wait states ahead of an asm block, so where y comes straight from
// a v_mfma result (no ordinary VALU instruction has read it first), AFTER_MFMA opens the
// block with 12 of them: gfx950 needs 8 between a 16x16x32 result and a VALU read.
#define RHTQ_SPLIT8_BODY                                                       \
  "v_fma_mixlo_f16 %0, %8, %16, 0\n\t"                                        \
  "v_fma_mixlo_f16 %1, %10, %16, 0\n\t"                                       \
  "v_fma_mixlo_f16 %2, %12, %16, 0\n\t"                                       \
  "v_fma_mixlo_f16 %3, %14, %16, 0\n\t"                                       \
  "v_fma_mixhi_f16 %0, %9, %16, 0\n\t"                                        \
  "v_fma_mixhi_f16 %1, %11, %16, 0\n\t"                                       \
  "v_fma_mixhi_f16 %2, %13, %16, 0\n\t"                                       \
  "v_fma_mixhi_f16 %3, %15, %16, 0\n\t"                                       \
  "v_fma_mixlo_f16 %4, %8, %16, -%0 op_sel_hi:[0,0,1]\n\t"                    \
  "v_fma_mixlo_f16 %5, %10, %16, -%1 op_sel_hi:[0,0,1]\n\t"                   \
  "v_fma_mixlo_f16 %6, %12, %16, -%2 op_sel_hi:[0,0,1]\n\t"                   \
  "v_fma_mixlo_f16 %7, %14, %16, -%3 op_sel_hi:[0,0,1]\n\t"                   \
  "v_fma_mixhi_f16 %4, %9, %16, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"     \
  "v_fma_mixhi_f16 %5, %11, %16, -%1 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"    \
  "v_fma_mixhi_f16 %6, %13, %16, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"    \
  "v_fma_mixhi_f16 %7, %15, %16, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"    \
  "s_nop 1"
template <bool AFTER_MFMA = false>
__device__ __forceinline__ void split8(const float* y, float S, uint32_t* hi, uint32_t* lo) {
  if constexpr (AFTER_MFMA) {
    asm("s_nop 7\n\ts_nop 3\n\t" RHTQ_SPLIT8_BODY
        : "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]), "=&v"(hi[3]),
          "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3])
        : "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]), "v"(y[4]), "v"(y[5]), "v"(y[6]), "v"(y[7]),
          "v"(S));
  } else {
    asm(RHTQ_SPLIT8_BODY
        : "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]), "=&v"(hi[3]),
          "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3])
        : "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]), "v"(y[4]), "v"(y[5]), "v"(y[6]), "v"(y[7]),
          "v"(S));
  }
}
#undef RHTQ_SPLIT8_BODY

// split8 with a scale of its own for each half: elements 0-3 under S0, elements 4-7 under S1
// (words 0-1 and 2-3 of hi / lo), for eight values drawn from two independent rows.
__device__ __forceinline__ void split8x2(const float* y, float S0, float S1, uint32_t* hi, uint32_t* lo) {
  asm("v_fma_mixlo_f16 %0, %8, %16, 0\n\t"
      "v_fma_mixlo_f16 %1, %10, %16, 0\n\t"
      "v_fma_mixlo_f16 %2, %12, %17, 0\n\t"
      "v_fma_mixlo_f16 %3, %14, %17, 0\n\t"
      "v_fma_mixhi_f16 %0, %9, %16, 0\n\t"
      "v_fma_mixhi_f16 %1, %11, %16, 0\n\t"
      "v_fma_mixhi_f16 %2, %13, %17, 0\n\t"
      "v_fma_mixhi_f16 %3, %15, %17, 0\n\t"
      "v_fma_mixlo_f16 %4, %8, %16, -%0 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %5, %10, %16, -%1 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %6, %12, %17, -%2 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %7, %14, %17, -%3 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %4, %9, %16, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %5, %11, %16, -%1 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %6, %13, %17, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %7, %15, %17, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]), "=&v"(hi[3]),
        "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3])
      : "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]), "v"(y[4]), "v"(y[5]), "v"(y[6]), "v"(y[7]),
        "v"(S0), "v"(S1));
}

// E4M3FN (OCP FP8) code of s >= 0: nearest value, ties to even mantissa, saturating at
// 448 (0x7E), subnormals kept; NaN never produced.  gfx950's conversion instruction does the
// rounding; the input is clamped to 448 first so nothing overflows.  Checked on the device
// against a bit-level definition of this encoding on every code, every midpoint between
// neighbouring codes (and one ulp either side) and 65536 log-uniform values: no difference.
__device__ __forceinline__ uint32_t e4m3_code(float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// Value of an E4M3FN code 0 .. 0x7E (the conversion instruction; exact).
__device__ __forceinline__ float e4m3_value(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// MX shared exponent of a 32-block with maximum bmax >= 0 (OCP MX v1.0): floor(log2(bmax))
// minus 2 (the largest E2M1 normal is 1.5 * 2^2), clamped to [-127, 127]; -127 for a zero
// block.  For a normal bmax the floor of log2 is its unbiased exponent field; a subnormal
// bmax is below 2^-126 and clamps.
__device__ __forceinline__ int mx_exponent(float bmax) {
  const int e = (int)((__float_as_uint(bmax) >> 23) & 0xFF) - 127 - 2;
  return bmax > 0.0f ? (e < -127 ? -127 : (e > 127 ? 127 : e)) : -127;
}

// NVFP4 tensor scale g = fl32(a / (6 * 448)) of a maximum a (correctly rounded division).
// Rounding is monotone, so the maximum of these over workgroups equals g of the overall
// maximum: the pre-pass combines per-workgroup values with an atomic max on the bits
// (non-negative floats order like their bit patterns) and leaves g itself.
__device__ __forceinline__ float nvfp4_tensor_scale(float a) { return a / 2688.0f; }

// Eight INT4 codes -> one dword, element k in nibble k.  q[k] holds the bits of
// fma(y, 1/s, 1.5 * 2^23): its low 4 bits are the two's-complement code.
__device__ __forceinline__ uint32_t pack8_nibbles(const uint32_t* q) {
  const uint32_t e_lo = __builtin_amdgcn_perm(q[2], q[0], 0x0C0C0400u);
  const uint32_t e_hi = __builtin_amdgcn_perm(q[6], q[4], 0x0C0C0400u);
  const uint32_t o_lo = __builtin_amdgcn_perm(q[3], q[1], 0x0C0C0400u);
  const uint32_t o_hi = __builtin_amdgcn_perm(q[7], q[5], 0x0C0C0400u);
  const uint32_t ev = __builtin_amdgcn_perm(e_hi, e_lo, 0x05040100u);   // bytes q0 q2 q4 q6
  const uint32_t od = __builtin_amdgcn_perm(o_hi, o_lo, 0x05040100u);   // bytes q1 q3 q5 q7
  return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}

}  // namespace rhtq
