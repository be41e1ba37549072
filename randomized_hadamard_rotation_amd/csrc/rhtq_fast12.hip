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
//     half t2 = h of the six sub-rows it lacks, in the other wave's units.
//  4. The order-12 Williamson factor in registers across the twelve sub-rows, taking the
//     received half into this wave's units on the way (or, where that half is far larger,
//     this wave's own half into the other wave's units, so that nothing is scaled up).
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
  float gmax[kW][kSub];                 // groups of whole sub-rows: each wave's group maxima
};

// INT4 groups of PER = 1, 2 or 4 whole sub-rows (1024, 2048 or 4096 elements).  A sub-row spans
// both waves (wave h holds its half 512 h + [0, 512)), so each wave reduces its share of every
// group over its lanes and the two shares meet in LDS, behind one barrier, as the per-token
// maximum does.  Chunk q of this wave is sub-row q; val and cbase as for quant_epilogue.
template <int PER, int H, typename ValF, typename BaseF>
__device__ __forceinline__ void fast12_whole_subrow_groups(const KernelArgs& a, Shared12& sh, const int64_t row,
                                                           const int64_t relem0, const float invS, const float cnorm,
                                                           const int lane, const int lc, ValF val, BaseF cbase) {
  constexpr int NGR = kSub / PER;   // groups per row
  float gm[NGR];
#pragma unroll
  for (int k = 0; k < NGR; ++k) {
    float m = 0.0f;
#pragma unroll
    for (int q = PER * k; q < PER * (k + 1); ++q)
#pragma unroll
      for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
    gm[k] = group_max(m, 64) * invS;   // this wave's half of group k, true units
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < NGR; ++k) sh.gmax[H][k] = gm[k];
  }
  __syncthreads();
  float inv[kSub];
  bool clamp = false;
#pragma unroll
  for (int k = 0; k < NGR; ++k) {
    const Int4Scale sc = int4_scale(fmaxf(sh.gmax[0][k], sh.gmax[1][k]), cnorm, a.scale_dtype);
    clamp |= sc.clamp;
#pragma unroll
    for (int q = PER * k; q < PER * (k + 1); ++q) inv[q] = sc.inv * invS;
    if (H == 0 && lane == 0) store_int4_scale(a.scales, a.scale_dtype, row * NGR + k, sc.s);
  }
  int4_codes<kSub>(a.packed + (relem0 >> 1), inv, clamp, lc, val, cbase);
}

// The order-12 factor (h12_forward) on values of which the other wave's six sub-rows are still in
// that wave's units: their factor rho (a power of two) enters the column sums once and otherwise
// rides on additions the array already needs, as fused multiply-adds, instead of one multiply per
// received value.  Scaling by a power of two is exact, so the results equal h12_forward of the
// rescaled values (each rounding step is the same one on a scaled operand).  Wave 0 owns blocks 0-1 (j1 < 6) and receives blocks 2-3, wave 1 the reverse.
template <int H>
__device__ __forceinline__ void h12_forward_rho(float* w, const float rho) {
  float s1 = w[0] + w[1] + w[2];
  float s2 = w[3] + w[4] + w[5];
  float s3 = w[6] + w[7] + w[8];
  float s4 = w[9] + w[10] + w[11];
  if constexpr (H == 0) { s3 *= rho; s4 *= rho; } else { s1 *= rho; s2 *= rho; }
  const float pa = s1 + s3, pb = s2 + s4, pc = s2 - s4, pd = s3 - s1;
  const float t1 = pa + pb, t2 = pb - pa, t3 = pc + pd, t4 = pd - pc;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const float v1 = w[k], v2 = w[3 + k], v3 = w[6 + k], v4 = w[9 + k];
    if constexpr (H == 0) {   // v3, v4 received
      const float s34 = v3 + v4, d34 = v3 - v4, s12 = v1 + v2;
      const float d24 = __builtin_fmaf(-rho, v4, v2);
      w[k] = __builtin_fmaf(-2.0f, __builtin_fmaf(rho, s34, v2), t1);     // -2 (v2 + v3 + v4)
      w[3 + k] = __builtin_fmaf(2.0f, __builtin_fmaf(rho, d34, v1), t2);  // +2 (v1 + v3 - v4)
      w[6 + k] = __builtin_fmaf(2.0f, v1 - d24, t3);                      // +2 (v1 - v2 + v4)
      w[9 + k] = __builtin_fmaf(2.0f, __builtin_fmaf(-rho, v3, s12), t4); // +2 (v1 + v2 - v3)
    } else {                  // v1, v2 received
      const float s34 = v3 + v4, d34 = v3 - v4, s12 = v1 + v2;
      const float d24 = __builtin_fmaf(rho, v2, -v4);
      w[k] = __builtin_fmaf(-2.0f, __builtin_fmaf(rho, v2, s34), t1);
      w[3 + k] = __builtin_fmaf(2.0f, __builtin_fmaf(rho, v1, d34), t2);
      w[6 + k] = __builtin_fmaf(2.0f, __builtin_fmaf(rho, v1, -d24), t3);
      w[9 + k] = __builtin_fmaf(2.0f, __builtin_fmaf(rho, s12, -v3), t4);
    }
  }
}

// Rows of the workgroup as seen by wave H (a template parameter, so that every register
// array is indexed by constants).  Both waves pass the same barriers in the same order.
template <int OP, int H, int PER, bool F32, bool H16>
__device__ __forceinline__ void fast12_rows(const KernelArgs& a, Shared12& sh, const bf16x8 (&hb)[2],
                                            const f16x8 (&hc)[2], const int lane, const float gts,
                                            const float inv6g, const int G) {
  constexpr int h = H, other = 1 - H;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)kN));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  float run_max = 0.0f;
  const int lc = (lane >> 4) | ((lane & 15) << 2);

  // loads of one row (12 x 16 bytes per lane); the next row's go out as soon as stage 1
  // has consumed these registers, so they run during this row's work.  fp32 input (F32):
  // 12 x 2 x 16 bytes per lane, loaded at the top of each row (no registers for a prefetch).
  uint4 raw[F32 ? 1 : kOwn][2] = {};
  uint4 raw32[F32 ? kOwn : 1][2][2] = {};
  const float* xf = static_cast<const float*>(a.x);
  auto load = [&](int64_t r) {
    if (r < a.rows) {
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          if constexpr (F32) {
            const float* p = xf + r * kN + load_off(h, jl, f, lane);
            raw32[jl][f][0] = ld_stream(p);
            raw32[jl][f][1] = ld_stream(p + 4);
          } else {
            raw[jl][f] = ld_stream(x + r * kN + load_off(h, jl, f, lane));
          }
        }
    }
  };
  if constexpr (!F32) load(blockIdx.x);

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t relem0 = row * kN;
    if constexpr (F32) load(row);
    // ---------------- H1024 of the own sub-rows ----------------
    float d1[kOwn][2][2][4];   // [jl][f][t][i]
#pragma unroll
    for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const uint4 mk = sh.sign_tab[((h * kOwn + jl) * 2 + f) * 64 + lane];
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 p0, p1;
        if constexpr (F32) {
          // three bf16 terms per value (split3_bf16); the signs flip each term
          uint32_t th[4], tm[4], tl[4];
          split3_bf16(raw32[jl][f][0], raw32[jl][f][1], th, tm, tl);
          const uint32_t m4[4] = {mk.x, mk.y, mk.z, mk.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) { th[k] ^= m4[k]; tm[k] ^= m4[k]; tl[k] ^= m4[k]; }
          bf16x8 ah, am, al;
          __builtin_memcpy(&ah, th, 16);
          __builtin_memcpy(&am, tm, 16);
          __builtin_memcpy(&al, tl, 16);
          p0 = stage1_f32(ah, am, al, hb[0]);
          p1 = stage1_f32(ah, am, al, hb[1]);
        } else {
          uint4 r = raw[jl][f];
          r.x ^= mk.x; r.y ^= mk.y; r.z ^= mk.z; r.w ^= mk.w;
          bf16x8 av;
          __builtin_memcpy(&av, &r, 16);
          p0 = stage1_mma<H16>(av, hb[0], z);
          p1 = stage1_mma<H16>(av, hb[1], z);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) { d1[jl][f][0][i] = p0[i]; d1[jl][f][1][i] = p1[i]; }
      }
    if constexpr (!F32) load(row + gridDim.x);
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
    float rho = 1.0f, xso = 1.0f;   // xso: the other wave's inverse split scale
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      __syncthreads();   // the other wave has read the previous contents of xbuf
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
        for (int i = 0; i < 4; ++i) sh.xbuf[h][jl * 4 + i][lane] = d2[jl][t][other][i];
      if (t == 0 && lane == 0) sh.xs[h] = invS;
      __syncthreads();
      if (t == 0) {
        xso = sh.xs[other];
        rho = S * xso;   // ratio of two powers of two: exact (or out of range, handled below)
      }
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[kOwn * other + jl][t][i] = sh.xbuf[other][jl * 4 + i][lane];
    }
    // rho takes the received half into this wave's units.  Where that half is far larger (rho
    // above 2^40; a dynamic range above about 2^108 between the halves would take it past fp32's
    // range), this wave works in the other wave's units instead: its own values go down by 1/rho
    // (a power of two, or to zero below fp32's range, far under the received half's rounding).
    // The branch is uniform.
    if (rho > 0x1p40f) {
      const float down = __builtin_amdgcn_rcpf(rho);
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) w[kOwn * h + jl][t][i] *= down;
      rho = 1.0f;
      invS = xso;
    }
    // keep the order-12 factor after both exchange steps: scheduled between them it lengthens the
    // stretch between barriers that the other wave waits on
    __builtin_amdgcn_sched_barrier(0);

    // ---------------- order-12 factor (the received half rescaled by rho on the way) ----------------
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v[kSub];
#pragma unroll
        for (int j1 = 0; j1 < kSub; ++j1) v[j1] = w[j1][t][i];
        h12_forward_rho<H>(v, rho);
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
      if constexpr (PER > 0) {   // INT4 groups of whole sub-rows
        (void)rowmax;
        fast12_whole_subrow_groups<PER, H>(a, sh, row, relem0, invS, cnorm, lane, lc, val, cbase);
      } else {
        quant_epilogue<OP, kSub>(a, row, relem0, G, invS, cnorm, gts, inv6g, lane, lane == 0 && h == 0, val,
                                 cbase, rowmax);
      }
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


// PER = 0: groups inside a wave's chunks (or per-token); PER = 1, 2, 4: INT4 groups of PER whole
// sub-rows (a separate instantiation, so the common kernel carries no code for them).  F32: fp32
// input (three bf16 terms per value); H16: fp16 input (stage 1 on the f16 matrix-core instruction).
template <int OP, int PER, bool F32 = false, bool H16 = false>
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
  const bf16x8 hb[2] = {h32_operand<H16>(lane, 0), h32_operand<H16>(lane, 1)};
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
  if (h == 0) fast12_rows<OP, 0, PER, F32, H16>(a, sh, hb, hc, lane, gts, inv6g, G);
  else fast12_rows<OP, 1, PER, F32, H16>(a, sh, hb, hc, lane, gts, inv6g, G);
}

template <int OP, int PER, int IN>
hipError_t launch12k(const KernelArgs& a, hipStream_t s) {
  auto kern = fast12_kernel<OP, PER, IN == RHTQ_IN_F32, IN == RHTQ_IN_F16>;
  static const int max_blocks = resident_blocks((const void*)kern, kT, 0);
  const int grid = (int)(a.rows < max_blocks ? a.rows : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kT), 0, s, a);
  return hipGetLastError();
}

template <int OP, int IN>
hipError_t launch12(const KernelArgs& a, hipStream_t s) {
  if (a.sign_period != kN) return hipErrorNotSupported;
  if constexpr (OP == OP_INT4) {
    // per-token, groups of 16 .. 512 inside a wave's chunks, or 1024 .. 4096 (whole sub-rows)
    if (!(a.group == kN || (a.group >= 16 && a.group <= 4096))) return hipErrorNotSupported;
    if (a.group == 1024) return launch12k<OP, 1, IN>(a, s);
    if (a.group == 2048) return launch12k<OP, 2, IN>(a, s);
    if (a.group == 4096) return launch12k<OP, 4, IN>(a, s);
  }
  return launch12k<OP, 0, IN>(a, s);
}

}  // namespace

int64_t fast12_grid(int64_t rows) {
  static const int max_blocks = resident_blocks((const void*)fast12_kernel<OP_INT4, 0, false>, kT, 0);
  return rows < max_blocks ? rows : max_blocks;
}

namespace {
template <int IN>
hipError_t launch12_op(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return launch12<OP_ROTATE, IN>(a, s);
    case OP_INT4: return launch12<OP_INT4, IN>(a, s);
    case OP_NVFP4: return launch12<OP_NVFP4, IN>(a, s);
    case OP_MXFP4: return launch12<OP_MXFP4, IN>(a, s);
    case OP_AMAX: return launch12<OP_AMAX, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}
}  // namespace

hipError_t launch_fast12(int op, const KernelArgs& a, hipStream_t s, bool f16in) {
  return f16in ? launch12_op<RHTQ_IN_F16>(op, a, s) : launch12_op<RHTQ_IN_BF16>(op, a, s);
}

hipError_t launch_fast12_f32(int op, const KernelArgs& a, hipStream_t s) {
  return launch12_op<RHTQ_IN_F32>(op, a, s);
}

}  // namespace rhtq
