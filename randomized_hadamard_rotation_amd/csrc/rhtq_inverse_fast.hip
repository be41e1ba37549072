// Inverse for KV-cache rows (head dim 64, 128 or 256) stored as INT4 with one scale per row:
// unpack, dequantise and undo the rotation, x = diag(s) H^T (q * scale) / sqrt(n).
// QuaRot reviews: review 2 Summary (the random Hadamard transform is invertible), review 3
// Strengths and reviewer 2 follow-up (the KV cache is rotated and quantised, then read back).
//
// The scale is constant over the row, so H^T (q * scale) = scale * (H q) and the transform runs
// on the integer codes themselves, exactly, on the int8 matrix cores:
//
//  1. Each lane loads 8 bytes = 16 codes of one 64-element block (one row of 16 lanes x 4 lane
//     groups covers 1024 codes, 512 bytes).  Each nibble c becomes the byte c ^ 8 = q + 8 (0..15),
//     the low nibbles of the two dwords then the high nibbles, one v_bitop3 per dword.
//  2. v_mfma_i32_16x16x64_i8 against a +-1 int8 H64 contracts index bits 0-5 in int32.  The
//     K-slot order of the operand is the unpack order above; A and B use the same slot-to-element
//     map, so the product is exact whatever order the hardware assigns to the slots.  The +8 bias
//     adds 8 * 64 to output 0 of each block only (the columns of H64 sum to zero except the first),
//     which one subtraction removes.
//  3. Index bits 6.. (128: one, 256: two) are int32 butterflies between registers.
//  4. fp32 conversion, multiplication by scale / sqrt(n) (the scales are loaded with the codes, so
//     no load follows a store in a wave step and the stores never wait), the random signs by XOR
//     of fp32 sign bits held in registers (a lane always serves the same columns), and 16-byte
//     stores: each wave store covers 256 contiguous bytes per row.
#include <hip/hip_fp16.h>

#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

constexpr int kWavesI = 4;
constexpr int kThreadsI = 64 * kWavesI;
constexpr int kUnit = 1024;   // codes per wave step

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Element of the 64-block held in K-slot e of a lane in lane group g (the unpack order).
__host__ __device__ constexpr int slot_element(int g, int e) { return 16 * g + (e < 8 ? 2 * e : 2 * (e - 8) + 1); }

// B operand for output tile tau: slot (lane >> 4, e) against column n = lane & 15, which stands
// for output element 4 n + tau of the 64-block.  Entries +1 / -1 as int8.
__device__ __forceinline__ i32x4 h64_i8_operand(int lane, int tau) {
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int k = slot_element(lane >> 4, e);
    const int o = 4 * (lane & 15) + tau;
    const uint32_t b = (__builtin_popcount(k & o) & 1) ? 0xFFu : 0x01u;
    w[e >> 2] |= b << (8 * (e & 3));
  }
  const i32x4 r = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  return r;
}

// SD: scale storage (RHTQ_SCALE_F32 / F16), a template parameter so that the scale loads of a
// wave step carry no branch and issue together with the codes
template <int L, int SD>
__global__ __launch_bounds__(kThreadsI) void inv_kv_kernel(KernelArgs a) {
  constexpr int N = 1 << L;
  constexpr int HB = L - 6;                 // index bits above the 64-block: 0, 1 or 2
  constexpr int RPU = kUnit / N;            // rows per wave step
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, n = lane & 15;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)N));

  i32x4 hb[4];
#pragma unroll
  for (int tau = 0; tau < 4; ++tau) hb[tau] = h64_i8_operand(lane, tau);
  // sign masks of the outputs this lane writes: element 64 hi + 4 n + tau
  uint32_t smask[1 << HB][4];
#pragma unroll
  for (int hi = 0; hi < (1 << HB); ++hi)
#pragma unroll
    for (int tau = 0; tau < 4; ++tau)
      smask[hi][tau] = (a.signs && a.signs[64 * hi + 4 * n + tau] < 0) ? 0x80000000u : 0u;
  const uint32_t bias = n == 0 ? 512u : 0u;   // 8 * 64 on output 0 of the block

  // this lane's 8 code bytes: row (lane & 15) >> HB of the step, 64-block (lane & 15) & mask
  const int m = lane & 15;
  const int lrow = m >> HB, lhi = m & ((1 << HB) - 1);
  const int load_off = lrow * (N / 2) + 32 * lhi + 8 * g;

  const int64_t units = (a.rows + RPU - 1) / RPU;
  for (int64_t u = (int64_t)blockIdx.x * kWavesI + wave; u < units; u += (int64_t)gridDim.x * kWavesI) {
    const int64_t row0 = u * RPU;
    // scales of the rows this lane stores, issued first and together with the codes: a load issued
    // after this unit's stores would wait for them (the memory counter is in order), once per row
    constexpr int RL = 4 >> HB;                // rows per lane: output rows (4 g + i) >> HB, i = 0..3
    float rs[RL];
#pragma unroll
    for (int k = 0; k < RL; ++k) {
      int64_t rr = row0 + ((4 * g) >> HB) + k;
      rr = rr < a.rows ? rr : a.rows - 1;      // in bounds; rows past the end are not stored
      if constexpr (SD == RHTQ_SCALE_F32) rs[k] = static_cast<const float*>(a.in_scales)[rr] * cnorm;
      else rs[k] = __half2float(static_cast<const __half*>(a.in_scales)[rr]) * cnorm;
    }
    u32x2 c = {0x88888888u, 0x88888888u};   // codes of absent rows: q = -8 (never stored)
    if (row0 + lrow < a.rows)
      c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a.in_packed + row0 * (N / 2) + load_off));
    // q + 8 = c ^ 8 per nibble: low nibbles of both dwords, then high nibbles
    i32x4 av;
    av.x = (int)((c.x & 0x0F0F0F0Fu) ^ 0x08080808u);
    av.y = (int)((c.y & 0x0F0F0F0Fu) ^ 0x08080808u);
    av.z = (int)(((c.x >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u);
    av.w = (int)(((c.y >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u);

    // d[tau][i]: row 4 g + i of the product (step row (4 g + i) >> HB, block (4 g + i) & mask),
    // output element 4 n + tau of the block
    int d[4][4];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
      const i32x4 z = {0, 0, 0, 0};
      const i32x4 p = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, hb[tau], z, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[tau][i] = p[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) d[0][i] -= (int)bias;
    // index bits 6.. : register index bits 0 .. HB-1
#pragma unroll
    for (int b = 0; b < HB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((i & (1 << b)) == 0)
#pragma unroll
          for (int tau = 0; tau < 4; ++tau) {
            const int s0 = d[tau][i], s1 = d[tau][i | (1 << b)];
            d[tau][i] = s0 + s1;
            d[tau][i | (1 << b)] = s0 - s1;
          }

    // the scales have arrived before the first store: a wait for them between the stores would
    // also wait for the stores already issued
    if constexpr (RL == 1) asm volatile("" ::"v"(rs[0]) : "memory");
    else if constexpr (RL == 2) asm volatile("" ::"v"(rs[0]), "v"(rs[1]) : "memory");
    else asm volatile("" ::"v"(rs[0]), "v"(rs[1]), "v"(rs[2]), "v"(rs[3]) : "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (4 * g + i) >> HB;       // row within the step
      const int hi = (4 * g + i) & ((1 << HB) - 1);
      const int64_t row = row0 + r;
      if (row >= a.rows) continue;
      const float s = rs[i >> HB];
      float o[4];
#pragma unroll
      for (int tau = 0; tau < 4; ++tau) o[tau] = __uint_as_float(__float_as_uint((float)d[tau][i] * s) ^ smask[hi][tau]);
      st_stream(a.y + row * N + 64 * hi + 4 * n, o[0], o[1], o[2], o[3]);
    }
  }
}

template <int L, int SD>
hipError_t launch_inv(const KernelArgs& a, hipStream_t s) {
  auto kern = inv_kv_kernel<L, SD>;
  static const int max_blocks = resident_blocks((const void*)kern, kThreadsI, 0);
  constexpr int RPU = kUnit / (1 << L);
  const int64_t units = (a.rows + RPU - 1) / RPU;
  const int64_t want = (units + kWavesI - 1) / kWavesI;
  const int grid = (int)(want < max_blocks ? want : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreadsI), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_inverse_fast(const KernelArgs& a, hipStream_t s) {
  if (a.inv_fmt != RHTQ_FMT_INT4 || a.group != a.n || a.sign_period != a.n) return hipErrorNotSupported;
  if (reinterpret_cast<uintptr_t>(a.in_packed) & 7) return hipErrorNotSupported;
  const bool f32 = a.scale_dtype == RHTQ_SCALE_F32;
  switch (a.n) {
    case 64: return f32 ? launch_inv<6, RHTQ_SCALE_F32>(a, s) : launch_inv<6, RHTQ_SCALE_F16>(a, s);
    case 128: return f32 ? launch_inv<7, RHTQ_SCALE_F32>(a, s) : launch_inv<7, RHTQ_SCALE_F16>(a, s);
    case 256: return f32 ? launch_inv<8, RHTQ_SCALE_F32>(a, s) : launch_inv<8, RHTQ_SCALE_F16>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace rhtq
