// Two-wavefront kernel for rows of 12288 = 12 x 1024 bf16 values (KronQ issue #2,
// Model Details: the 12288-wide intermediate activation is 12 x 1024,
// Hadamard-compatible; QuaRot reviews, review 2 Questions: non-power-of-two widths
// need an extra factor next to the power-of-two transform).
//
// Index j = 1024 j1 + j2 (j1 < 12, j2 < 1024); H_12288 = H12 (x) H1024.  The two waves
// of a workgroup share one row: wave h holds the half j2 bit 9 = h of all twelve
// sub-rows (96 values per lane), which keeps the per-lane state low enough for two
// waves per SIMD.  Per row:
//
//  1. 16-byte loads in the MFMA A layout (element 1024 j1 + 512 h + 32 (l & 15) +
//     8 (l >> 4) + e), random signs by XOR with bf16 sign masks from an LDS table.
//  2. Bits 0-4 of j2 on v_mfma_f32_16x16x32_bf16 against the +-1 H32 operand.
//  3. Bits 5-6 in registers; bits 7-8 through v_permlane16/32_swap and registers.
//  4. The order-12 Williamson factor across the twelve sub-rows, in registers.
//  5. Bit 9 couples the two waves: each sub-row is exchanged through a double-buffered
//     LDS chunk; wave h reads the element pairs (j2, j2 + 512) of its own output half
//     (8 consecutive j2 per lane) and forms a + b (h = 0) or a - b (h = 1).  The same
//     pass leaves 8 consecutive outputs per lane for the epilogue.
//  6. Epilogue as in the other fast kernels: group maxima by DPP, INT4 magic-constant
//     rounding or E2M1 conversion, packed 4-byte stores.
#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

constexpr int kW = 2;              // waves per workgroup (one row)
constexpr int kT = 64 * kW;
constexpr int kN = 12288;
constexpr int kSub = 12;           // sub-rows of 1024
constexpr int kTB = 1024 + 128;    // padded chunk buffer (floats)

// 4 padding floats after every 32: the 8-byte pair stores and the 16-byte reads of
// 8 consecutive floats per lane then touch distinct LDS banks
__device__ __forceinline__ int tp(int j) { return j + ((j >> 5) << 2); }

// element offset (within a row) of this lane's 8 loaded values of sub-row j1
__device__ __forceinline__ int load_off(int j1, int h, int lane) {
  return 1024 * j1 + 512 * h + 32 * (lane & 15) + 8 * (lane >> 4);
}

template <int OP>
__global__ __launch_bounds__(kT) void fast12_kernel(KernelArgs a) {
  __shared__ float tbuf[2][kTB];
  __shared__ float rowmax[kW];
  __shared__ uint4 sign_tab[kSub * kW * 64];   // bf16 sign-bit masks in load order
  const int lane = threadIdx.x & 63;
  const int h = threadIdx.x >> 6;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)kN));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);

  // bf16 sign-bit masks in load order: entry (j1 * 2 + h) * 64 + lane covers the 8 elements
  // that lane loads for sub-row j1 in wave h, so the table reads are conflict-free
  for (int k = threadIdx.x; k < kSub * kW * 64; k += kT) {
    uint4 m = make_uint4(0, 0, 0, 0);
    if (a.signs) {
      const uint2 sv = *reinterpret_cast<const uint2*>(a.signs + load_off(k >> 7, (k >> 6) & 1, k & 63));
      m.x = __builtin_amdgcn_perm(0u, sv.x, 0x010C000Cu) & 0x80008000u;
      m.y = __builtin_amdgcn_perm(0u, sv.x, 0x030C020Cu) & 0x80008000u;
      m.z = __builtin_amdgcn_perm(0u, sv.y, 0x010C000Cu) & 0x80008000u;
      m.w = __builtin_amdgcn_perm(0u, sv.y, 0x030C020Cu) & 0x80008000u;
    }
    sign_tab[k] = m;
  }
  __syncthreads();
  const bf16x8 hb[2] = {h32_operand(lane, 0), h32_operand(lane, 1)};
  float gts = 0.0f, inv6g = 0.0f;
  if constexpr (OP == OP_NVFP4) {
    gts = a.tensor_scale[0];
    inv6g = gts > 0.0f ? 1.0f / (6.0f * gts) : 0.0f;
  }
  const int group = a.group;
  float run_max = 0.0f;

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t rbase = row * kN;
    float v[kSub][2][4];
#pragma unroll
    for (int j1 = 0; j1 < kSub; ++j1) {
      uint4 r = ld_stream(x + rbase + load_off(j1, h, lane));
      const uint4 mk = sign_tab[(j1 * kW + h) * 64 + lane];
      r.x ^= mk.x; r.y ^= mk.y; r.z ^= mk.z; r.w ^= mk.w;
      bf16x8 av;
      __builtin_memcpy(&av, &r, 16);
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb[0], z, 0, 0, 0);
      const f32x4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb[1], z, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[j1][0][i] = d0[i]; v[j1][1][i] = d1[i]; }
    }
    // bits 5, 6 (register index i)
#pragma unroll
    for (int j1 = 0; j1 < kSub; ++j1)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bfly(v[j1][t][0], v[j1][t][1]);
        bfly(v[j1][t][2], v[j1][t][3]);
        bfly(v[j1][t][0], v[j1][t][2]);
        bfly(v[j1][t][1], v[j1][t][3]);
      }
    // order-12 factor across the sub-rows
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float w[kSub];
#pragma unroll
        for (int j1 = 0; j1 < kSub; ++j1) w[j1] = v[j1][t][i];
        h12_forward(w);
#pragma unroll
        for (int j1 = 0; j1 < kSub; ++j1) v[j1][t][i] = w[j1];
      }
    // bits 7, 8 (lane bits 4, 5) exchanged with register bits 5, 6
#pragma unroll
    for (int j1 = 0; j1 < kSub; ++j1)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j1][t][i]),
                                                    __float_as_uint(v[j1][t][i + 1]), false, false);
          v[j1][t][i] = __uint_as_float(p[0]);
          v[j1][t][i + 1] = __uint_as_float(p[1]);
          bfly(v[j1][t][i], v[j1][t][i + 1]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j1][t][i]),
                                                    __float_as_uint(v[j1][t][i + 2]), false, false);
          v[j1][t][i] = __uint_as_float(p[0]);
          v[j1][t][i + 2] = __uint_as_float(p[1]);
          bfly(v[j1][t][i], v[j1][t][i + 2]);
        }
      }
    // Element of (j1, t, i) now: j2 = 512 h + 128 i + 32 (lane >> 4) + 2 (lane & 15) + t.

    // bit 9: exchange each sub-row through LDS; this wave keeps j2 = 512 h + 8 lane + r
    float yo[kSub][8];
#pragma unroll
    for (int c = 0; c < kSub; ++c) {
      float* buf = tbuf[c & 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jl = 512 * h + 128 * i + 32 * (lane >> 4) + 2 * (lane & 15);
        *reinterpret_cast<float2*>(buf + tp(jl)) = make_float2(v[c][0][i], v[c][1][i]);
      }
      __syncthreads();
      const float4 lo0 = *reinterpret_cast<const float4*>(buf + tp(8 * lane));
      const float4 lo1 = *reinterpret_cast<const float4*>(buf + tp(8 * lane + 4));
      const float4 up0 = *reinterpret_cast<const float4*>(buf + tp(512 + 8 * lane));
      const float4 up1 = *reinterpret_cast<const float4*>(buf + tp(512 + 8 * lane + 4));
      const float sg = h == 0 ? 1.0f : -1.0f;
      yo[c][0] = __builtin_fmaf(sg, up0.x, lo0.x);
      yo[c][1] = __builtin_fmaf(sg, up0.y, lo0.y);
      yo[c][2] = __builtin_fmaf(sg, up0.z, lo0.z);
      yo[c][3] = __builtin_fmaf(sg, up0.w, lo0.w);
      yo[c][4] = __builtin_fmaf(sg, up1.x, lo1.x);
      yo[c][5] = __builtin_fmaf(sg, up1.y, lo1.y);
      yo[c][6] = __builtin_fmaf(sg, up1.z, lo1.z);
      yo[c][7] = __builtin_fmaf(sg, up1.w, lo1.w);
    }

    if constexpr (OP == OP_AMAX) {
#pragma unroll
      for (int c = 0; c < kSub; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r) run_max = fmaxf(run_max, fabsf(yo[c][r]));
      continue;
    }

    // per-token INT4: maximum of the whole row across both waves
    Int4Scale row_sc{0.0f, 0.0f, false};
    const bool row_group = (OP == OP_INT4) && (group == kN);
    if (row_group) {
      float m = 0.0f;
#pragma unroll
      for (int c = 0; c < kSub; ++c)
#pragma unroll
        for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(yo[c][r]));
      m = group_max(m, 64);
      if (lane == 0) rowmax[h] = m;
      __syncthreads();
      row_sc = int4_scale(fmaxf(rowmax[0], rowmax[1]), cnorm, a.scale_dtype);
    }

#pragma unroll
    for (int c = 0; c < kSub; ++c) {
      const int64_t g0 = rbase + 1024 * c + 512 * h + 8 * lane;   // first element of this lane
      if constexpr (OP == OP_ROTATE) {
        st_stream(a.y + g0, yo[c][0] * cnorm, yo[c][1] * cnorm, yo[c][2] * cnorm, yo[c][3] * cnorm);
        st_stream(a.y + g0 + 4, yo[c][4] * cnorm, yo[c][5] * cnorm, yo[c][6] * cnorm, yo[c][7] * cnorm);
      } else if constexpr (OP == OP_INT4) {
        Int4Scale sc = row_sc;
        int lpg = 64;
        if (!row_group) {
          float m = 0.0f;
#pragma unroll
          for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(yo[c][r]));
          lpg = group >> 3;
          sc = int4_scale(group_max(m, lpg), cnorm, a.scale_dtype);
        }
        uint32_t qb[8];
        if (__builtin_amdgcn_ballot_w64(sc.clamp) == 0) {
#pragma unroll
          for (int r = 0; r < 8; ++r) qb[r] = __float_as_uint(__builtin_fmaf(yo[c][r], sc.inv, 12582912.0f));
        } else {
#pragma unroll
          for (int r = 0; r < 8; ++r)
            qb[r] = __float_as_uint(__builtin_amdgcn_fmed3f(yo[c][r] * sc.inv, -8.0f, 7.0f) + 12582912.0f);
        }
        st_stream(a.packed + (g0 >> 1), pack8_nibbles(qb));
        const bool writer = row_group ? (c == 0 && h == 0 && lane == 0) : ((lane & (lpg - 1)) == 0);
        if (writer) {
          const int64_t gi = row_group ? row : (g0 >> __builtin_ctz((unsigned)group));
          if (a.scale_dtype == RHTQ_SCALE_F32) static_cast<float*>(a.scales)[gi] = sc.s;
          else static_cast<__half*>(a.scales)[gi] = __float2half_rn(fminf(sc.s, 65504.0f));
        }
      } else if constexpr (OP == OP_NVFP4) {
        // 16-element blocks over two lanes
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(yo[c][r]));
        m = group_max(m, 2);
        const uint32_t code = e4m3_code((m * cnorm) * inv6g);
        const float seff = e4m3_value(code) * gts;
        const float inv = seff > 0.0f ? cnorm * __builtin_amdgcn_rcpf(seff) : 0.0f;
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, yo[c][0] * inv, yo[c][1] * inv, 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, yo[c][2] * inv, yo[c][3] * inv, 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, yo[c][4] * inv, yo[c][5] * inv, 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, yo[c][6] * inv, yo[c][7] * inv, 1.0f, 3);
        st_stream(a.packed + (g0 >> 1), seff > 0.0f ? w : 0u);   // zero-scale block -> code 0
        if ((lane & 1) == 0) static_cast<uint8_t*>(a.scales)[g0 >> 4] = (uint8_t)code;
      }
    }
  }

  if constexpr (OP == OP_AMAX) {
    run_max = group_max(run_max, 64);
    if (lane == 0) rowmax[h] = run_max;
    __syncthreads();
    if (threadIdx.x == 0)
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale),
                __float_as_uint(fmaxf(rowmax[0], rowmax[1]) * cnorm));
  }
}

template <int OP>
hipError_t launch12(const KernelArgs& a, hipStream_t s) {
  if constexpr (OP == OP_INT4) {
    if (!(a.group == kN || a.group <= 512)) return hipErrorNotSupported;
  }
  auto kern = fast12_kernel<OP>;
  static const int max_blocks = [&] {
    int dev = 0, cus = 256, per_cu = 1;
    if (hipGetDevice(&dev) == hipSuccess)
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, kT, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    return cus * per_cu;
  }();
  const int64_t want = a.rows;
  const int grid = (int)(want < max_blocks ? want : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fast12(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return launch12<OP_ROTATE>(a, s);
    case OP_INT4: return launch12<OP_INT4>(a, s);
    case OP_NVFP4: return launch12<OP_NVFP4>(a, s);
    case OP_AMAX: return launch12<OP_AMAX>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace rhtq
