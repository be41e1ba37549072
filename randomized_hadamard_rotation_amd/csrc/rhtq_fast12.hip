// Two-wavefront kernel for rows of 12288 = 12 x 1024 bf16 values (KronQ issue #2,
// Model Details: the 12288-wide intermediate activation is 12 x 1024,
// Hadamard-compatible; QuaRot reviews, review 2 Questions: non-power-of-two widths
// need an extra factor next to the power-of-two transform).
//
// Index j = 1024 j1 + j2 (j1 < 12, j2 < 1024); H_12288 = H12 (x) H1024 and the factors
// commute.  The two waves of a workgroup share one row; wave h holds the sub-rows
// j1 = 6h .. 6h + 5 (96 values per lane).  Per row:
//
//  1. 16-byte loads in the MFMA A layout, random signs by XOR of bf16 sign bits.
//  2. H1024 of each sub-row on the matrix cores, as in the 1024..4096 kernel: bits 0-4 on
//     v_mfma_f32_16x16x32_bf16, bits 5-9 on v_mfma_f32_16x16x32_f16 with every value
//     split into two f16 terms under a power-of-two scale S.  Afterwards the lane holds,
//     per sub-row and per half t2 = j2 bit 9, eight consecutive outputs.
//  3. Exchange through LDS: wave h keeps the half t2 = h of every sub-row, so it sends
//     its other half (48 values per lane, in two steps) and receives the other wave's
//     half t2 = h of the six sub-rows it lacks, rescaled to its own S.
//  4. The order-12 Williamson factor in registers across the twelve sub-rows.
//  5. Epilogue on the twelve 512-element chunks 1024 j1 + 512 h + [0, 512): group
//     maxima, scales, INT4 or E2M1 codes, packed stores straight from registers.
#include <hip/hip_fp16.h>

#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_epilogue.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

constexpr int kW = 2;              // waves per workgroup (one row)
constexpr int kT = 64 * kW;
constexpr int kN = 12288;
constexpr int kSub = 12;           // sub-rows of 1024
constexpr int kOwn = 6;            // sub-rows per wave
constexpr int kX = kOwn * 4;       // values per lane in one exchange step

// element offset (within a row) of the 8 values this lane loads for own sub-row jl, fragment f
__device__ __forceinline__ int load_off(int h, int jl, int f, int lane) {
  return 1024 * (kOwn * h + jl) + 512 * f + 32 * (lane & 15) + 8 * (lane >> 4);
}

struct Shared12 {
  uint4 sign_tab[kW * kOwn * 2 * 64];   // bf16 sign-bit masks in load order
  float xbuf[kW][kX][64];               // exchange buffer, one step of each wave
  float xs[kW];                         // inverse split scale of each wave
  float rmax[kW];                       // per-token row maximum of each wave
};

// Rows of the workgroup as seen by wave H (a template parameter, so that every register
// array is indexed by constants).  Both waves pass the same barriers in the same order.
template <int OP, int H>
__device__ __forceinline__ void fast12_rows(const KernelArgs& a, Shared12& sh, const bf16x8 (&hb)[2],
                                            const f16x8 (&hc)[2], const int lane, const float gts,
                                            const float inv6g, const int G) {
  constexpr int h = H, other = 1 - H;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)kN));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  float run_max = 0.0f;
  const int lc = (lane >> 4) | ((lane & 15) << 2);

  // loads of one row (12 x 16 bytes per lane); the next row's go out as soon as stage 1
  // has consumed these registers, so they run during this row's work
  uint4 raw[kOwn][2] = {};
  auto load = [&](int64_t r) {
    if (r < a.rows) {
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
        for (int f = 0; f < 2; ++f) raw[jl][f] = ld_stream(x + r * kN + load_off(h, jl, f, lane));
    }
  };
  load(blockIdx.x);

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t relem0 = row * kN;
    // ---------------- H1024 of the own sub-rows ----------------
    float d1[kOwn][2][2][4];   // [jl][f][t][i]
#pragma unroll
    for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        uint4 r = raw[jl][f];
        const uint4 mk = sh.sign_tab[((h * kOwn + jl) * 2 + f) * 64 + lane];
        r.x ^= mk.x; r.y ^= mk.y; r.z ^= mk.z; r.w ^= mk.w;
        bf16x8 av;
        __builtin_memcpy(&av, &r, 16);
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        const f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb[0], z, 0, 0, 0);
        const f32x4 p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hb[1], z, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) { d1[jl][f][0][i] = p0[i]; d1[jl][f][1][i] = p1[i]; }
      }
    load(row + gridDim.x);
    float m1 = 0.0f;
#pragma unroll
    for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) m1 = fmaxf(m1, fabsf(d1[jl][f][t][i]));
    m1 = group_max(m1, 64);
    float S, invS;
    split_scale(__float_as_uint(m1), S, invS);

    // d2[jl][t][t2][i2]: element 1024 j1 + 512 t2 + 8 lc + t + 2 i2
    float d2[kOwn][2][2][4];
#pragma unroll
    for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float ys[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ys[e] = d1[jl][e >> 2][t][e & 3];
        uint32_t hw[4], lw[4];
        split8(ys, S, hw, lw);
        f16x8 ah, al;
        __builtin_memcpy(&ah, hw, 16);
        __builtin_memcpy(&al, lw, 16);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
          f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, hc[t2], z, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, hc[t2], acc, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) d2[jl][t][t2][i] = acc[i];
        }
      }

    // ---------------- exchange the halves ----------------
    // w[j1][t][i2]: the twelve sub-rows at this wave's half t2 = h, in this wave's units
    float w[kSub][2][4];
#pragma unroll
    for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[kOwn * h + jl][t][i] = d2[jl][t][h][i];
    float rho = 1.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      __syncthreads();   // the other wave has read the previous contents of xbuf
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
        for (int i = 0; i < 4; ++i) sh.xbuf[h][jl * 4 + i][lane] = d2[jl][t][other][i];
      if (t == 0 && lane == 0) sh.xs[h] = invS;
      __syncthreads();
      if (t == 0) rho = S * sh.xs[other];   // ratio of two powers of two: exact
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[kOwn * other + jl][t][i] = sh.xbuf[other][jl * 4 + i][lane] * rho;
    }

    // ---------------- order-12 factor ----------------
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v[kSub];
#pragma unroll
        for (int j1 = 0; j1 < kSub; ++j1) v[j1] = w[j1][t][i];
        h12_forward(v);
#pragma unroll
        for (int j1 = 0; j1 < kSub; ++j1) w[j1][t][i] = v[j1];
      }

    // chunk q = j1: elements 1024 q + 512 h + 8 lc + r
    auto val = [&](int q, int r) -> float { return w[q][r & 1][r >> 1]; };
    auto cbase = [&](int q) -> int { return 1024 * q + 512 * h; };

    if constexpr (OP == OP_AMAX) {
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < kSub; ++q)
#pragma unroll
        for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
      run_max = fmaxf(run_max, m * invS);
    } else if constexpr (OP == OP_ROTATE) {
#pragma unroll
      for (int q = 0; q < kSub; ++q) {
        float o[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) o[r] = (val(q, r) * invS) * cnorm;
        float* p = a.y + relem0 + cbase(q) + 8 * lc;
        st_stream(p, o[0], o[1], o[2], o[3]);
        st_stream(p + 4, o[4], o[5], o[6], o[7]);
      }
    } else {
      // per-token INT4: maximum of the whole row across both waves (uniform branch)
      auto rowmax = [&](float m) -> float {
        m = group_max(m, 64);
        if (lane == 0) sh.rmax[h] = m;
        __syncthreads();
        return fmaxf(sh.rmax[0], sh.rmax[1]);
      };
      quant_epilogue<OP, kSub>(a, row, relem0, G, invS, cnorm, gts, inv6g, lane, lane == 0 && h == 0, val,
                               cbase, rowmax);
    }
  }

  if constexpr (OP == OP_AMAX) {
    run_max = group_max(run_max, 64);
    if (lane == 0) sh.rmax[h] = run_max;
    __syncthreads();
    if (h == 0 && lane == 0)
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale), __float_as_uint(nvfp4_tensor_scale(fmaxf(sh.rmax[0], sh.rmax[1]) * cnorm)));
  }
}


template <int OP>
__global__ __launch_bounds__(kT) void fast12_kernel(KernelArgs a) {
  __shared__ Shared12 sh;
  const int lane = threadIdx.x & 63;
  const int h = threadIdx.x >> 6;

  for (int k = threadIdx.x; k < kW * kOwn * 2 * 64; k += kT) {
    uint4 m = make_uint4(0, 0, 0, 0);
    if (a.signs) {
      const int kl = k & 63, f = (k >> 6) & 1, jl = (k >> 7) % kOwn, hh = (k >> 7) / kOwn;
      const uint2 sv = *reinterpret_cast<const uint2*>(a.signs + load_off(hh, jl, f, kl));
      m.x = __builtin_amdgcn_perm(0u, sv.x, 0x010C000Cu) & 0x80008000u;
      m.y = __builtin_amdgcn_perm(0u, sv.x, 0x030C020Cu) & 0x80008000u;
      m.z = __builtin_amdgcn_perm(0u, sv.y, 0x010C000Cu) & 0x80008000u;
      m.w = __builtin_amdgcn_perm(0u, sv.y, 0x030C020Cu) & 0x80008000u;
    }
    sh.sign_tab[k] = m;
  }
  const bf16x8 hb[2] = {h32_operand(lane, 0), h32_operand(lane, 1)};
  const f16x8 hc[2] = {h32_stage2_operand(lane, 0), h32_stage2_operand(lane, 1)};
  __syncthreads();

  float gts = 0.0f, inv6g = 0.0f;
  if constexpr (OP == OP_NVFP4) {
    gts = a.tensor_scale[0];
    inv6g = gts > 0.0f ? 1.0f / (6.0f * gts) : 0.0f;
  }
  int G = 0;   // log2 of the INT4 group (0: one group per row)
  if constexpr (OP == OP_INT4) G = a.group == kN ? 0 : __builtin_ctz((unsigned)a.group);
  if constexpr (OP == OP_NVFP4) G = 4;
  if constexpr (OP == OP_MXFP4) G = 5;
  if (h == 0) fast12_rows<OP, 0>(a, sh, hb, hc, lane, gts, inv6g, G);
  else fast12_rows<OP, 1>(a, sh, hb, hc, lane, gts, inv6g, G);
}

template <int OP>
hipError_t launch12(const KernelArgs& a, hipStream_t s) {
  if (a.sign_period != kN) return hipErrorNotSupported;
  if constexpr (OP == OP_INT4) {
    if (!(a.group == kN || (a.group >= 16 && a.group <= 512))) return hipErrorNotSupported;
  }
  auto kern = fast12_kernel<OP>;
  static const int max_blocks = resident_blocks((const void*)kern, kT, 0);
  const int grid = (int)(a.rows < max_blocks ? a.rows : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fast12(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return launch12<OP_ROTATE>(a, s);
    case OP_INT4: return launch12<OP_INT4>(a, s);
    case OP_NVFP4: return launch12<OP_NVFP4>(a, s);
    case OP_MXFP4: return launch12<OP_MXFP4>(a, s);
    case OP_AMAX: return launch12<OP_AMAX>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace rhtq
