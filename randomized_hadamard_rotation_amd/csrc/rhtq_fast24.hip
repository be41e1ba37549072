// Four-wavefront kernel for rows of 24576 = 12 x 2048 bf16 values (KronQ issue #2,
// Model Details: a width of 12 times a power of two is Hadamard-compatible through the
// order-12 factor; QuaRot reviews, review 2 Questions: the non-power-of-two factor sits
// next to the power-of-two transform).
//
// Index j = 2048 j1 + j2 (j1 < 12, j2 < 2048); H_24576 = H12 (x) H2048 and the factors
// commute.  The four waves of a workgroup share one row; wave h holds the sub-rows
// j1 = 3h .. 3h + 2 (96 values per lane).  Per row:
//
//  1. 16-byte loads in the MFMA A layout, issued during the previous row's exchange (all
//     three sub-rows for rotate, MXFP4 and the amax pass; one for INT4 and NVFP4, the rest at
//     the top of the row); random signs by XOR of bf16 sign bits, the masks built per row from
//     the lane's own 96 sign bits (three registers).
//  2. Bits 0-4 of every 512-element fragment on v_mfma_f32_16x16x32_bf16.  The row's largest
//     stage-1 value over all four waves (first barrier) sets one power-of-two split scale S;
//     that pass keeps only the maximum, and each sub-row's stage 1 runs again before its split.
//  3. Bits 5-9 on v_mfma_f32_16x16x32_f16 with every value split into two f16 terms under S,
//     then bit 10 as a register butterfly between the two 1024-halves of each sub-row.  The
//     lane then holds, per sub-row and quarter q = j2 >> 9, eight consecutive outputs
//     512 q + 8 lc + e: the quarter is a register index.
//  4. Quarter q belongs to wave q.  Every lane keeps its own quarter in registers and writes
//     the other three to LDS for their waves at its own lane position, so the exchange needs
//     no lane permutation and stays bank-conflict free.  It takes two exchanges (three barriers)
//     to keep the workgroup within 64 KiB of LDS.
//  5. Each wave reads the nine sub-rows of its quarter computed by the other waves, applies
//     the order-12 Williamson factor across the twelve sub-rows, and runs the shared epilogue
//     on the twelve 512-element chunks 2048 j1 + 512 h + [0, 512).
#include <hip/hip_fp16.h>

#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_epilogue.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

constexpr int kW = 4;              // waves per workgroup (one row)
constexpr int kT = 64 * kW;
constexpr int kN = 24576;
constexpr int kM = 2048;           // sub-row length
constexpr int kSub = 12;           // sub-rows
constexpr int kOwn = 3;            // sub-rows per wave
constexpr int kNF = kM / 512;      // stage-1 fragments per sub-row

// element offset (within a row) of the 8 values this lane loads for own sub-row jl, fragment f
__device__ __forceinline__ int load_off(int h, int jl, int f, int lane) {
  return kM * (kOwn * h + jl) + 512 * f + 32 * (lane & 15) + 8 * (lane >> 4);
}

// LDS stays within 64 KiB per workgroup: the exchange moves 72 KiB per row, so it takes two
// exchange rounds.  The first carries the quarters for the waves d = 1 and 2 behind the sender (slot
// d - 1); the second reuses slot 0 for d = 3.
struct Shared24 {
  float4 xb[2][kW][kOwn][2][64];   // [slot][receiving wave][jl][half of the run][lane]
  float m1[kW];                    // stage-1 maximum of each wave
  float rmax[kW];                  // per-token row maximum of each wave
  float cmax[kW][kSub];            // INT4 groups above 512: each wave's chunk maxima
};

// INT4 groups of 2^(9 + BIG) elements (BIG = 1 .. 4: 1024 .. 8192).  Wave H holds chunk q =
// 2048 q + 512 H + [0, 512) of every sub-row q, so every such group spans two or four waves (and
// from 4096 on, several sub-rows): each wave reduces its chunks over its lanes, the maxima meet
// in LDS behind one barrier, and every wave takes its groups' maxima from there; the chunk that
// starts a group stores its scale.  val and cbase as for quant_epilogue.
template <int BIG, int H, typename ValF, typename BaseF>
__device__ __forceinline__ void fast24_big_groups(const KernelArgs& a, Shared24& sh, const int64_t row,
                                                  const int64_t relem0, const float invS, const float cnorm,
                                                  const int lane, const int lc, ValF val, BaseF cbase) {
  constexpr int G = 9 + BIG;
  float cm[kSub];
#pragma unroll
  for (int q = 0; q < kSub; ++q) {
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
    cm[q] = group_max(m, 64) * invS;
  }
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < kSub; ++q) sh.cmax[H][q] = cm[q];
  }
  __syncthreads();
  float inv[kSub];
  bool clamp = false;
#pragma unroll
  for (int q = 0; q < kSub; ++q) {
    // the group's chunks: sub-rows q0 .. q0 + nq - 1, waves h0 .. h0 + nh - 1
    constexpr int nq = G <= 11 ? 1 : 1 << (G - 11), nh = G == 10 ? 2 : 4;
    const int q0 = q & ~(nq - 1), h0 = G == 10 ? (H & 2) : 0;
    float m = 0.0f;
#pragma unroll
    for (int dq = 0; dq < nq; ++dq)
#pragma unroll
      for (int dh = 0; dh < nh; ++dh) m = fmaxf(m, sh.cmax[h0 + dh][q0 + dq]);
    const Int4Scale sc = int4_scale(m, cnorm, a.scale_dtype);
    clamp |= sc.clamp;
    inv[q] = sc.inv * invS;
    const int e = kM * q + 512 * H;   // the chunk's first element
    if (lane == 0 && (e & ((1 << G) - 1)) == 0) store_int4_scale(a.scales, a.scale_dtype, (relem0 + e) >> G, sc.s);
  }
  int4_codes<kSub>(a.packed + (relem0 >> 1), inv, clamp, lc, val, cbase);
}

// Sign bits of one own sub-row, one word per lane: the value the lane loads as element e of
// fragment f (dword k = e >> 1 of the 16-byte load) has its bit at 4 f + k, plus 16 for the
// odd element, so dword k's bf16 sign-bit mask is one shift and one AND away.
__device__ __forceinline__ uint32_t pack_signs(const int8_t* signs, int h, int jl, int lane) {
  uint32_t b = 0;
  if (signs) {
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const uint2 sv = *reinterpret_cast<const uint2*>(signs + load_off(h, jl, f, lane));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t byte = ((e < 4 ? sv.x : sv.y) >> (8 * (e & 3))) & 0xFFu;
        b |= (byte >> 7) << (4 * f + (e >> 1) + 16 * (e & 1));
      }
    }
  }
  return b;
}

// bf16 sign-bit masks of the 8 values of fragment f
__device__ __forceinline__ uint4 sign_masks(uint32_t b, int f) {
  uint4 m;
  m.x = (b << (15 - 4 * f)) & 0x80008000u;
  m.y = (b << (14 - 4 * f)) & 0x80008000u;
  m.z = (b << (13 - 4 * f)) & 0x80008000u;
  m.w = (b << (12 - 4 * f)) & 0x80008000u;
  return m;
}

// Bits 0-4 of 8 signed inputs (bf16, or fp16 when H16) against the H32 operand of one output
// half (exact).
template <bool H16>
__device__ __forceinline__ f32x4 stage1(const uint4& r, const bf16x8& hbt) {
  bf16x8 av;
  __builtin_memcpy(&av, &r, 16);
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  return stage1_mma<H16>(av, hbt, z);
}

// Rows of the workgroup as seen by wave H (a template parameter, so that every register
// array is indexed by constants).  All four waves pass the same barriers in the same order.
// F32: fp32 input.  Each value is split into three exact bf16 terms for stage 1 (split3_bf16,
// stage1_f32); the registers cannot hold the fp32 sub-rows between the two stage-1 passes, so
// each pass loads its sub-row when it needs it (no prefetch).
template <int OP, int H, bool H16, int BIG, bool F32>
__device__ __forceinline__ void fast24_rows(const KernelArgs& a, Shared24& sh, const bf16x8 (&hb)[2],
                                            const f16x8 (&hc)[2], const uint32_t (&sb)[kOwn], const int lane,
                                            const float gts, const float inv6g, const int G) {
  constexpr int h = H;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)kN));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  float run_max = 0.0f;
  const int lc = (lane >> 4) | ((lane & 15) << 2);

  // sub-rows loaded one row ahead: all three, except for INT4 and NVFP4, whose epilogues
  // leave registers for one (the others are loaded at the top of their own row)
  constexpr int kPf = (OP == OP_INT4 || OP == OP_NVFP4) ? 1 : kOwn;
  uint4 raw[kOwn][kNF] = {};
  auto load = [&](int64_t r, int j0, int j1) {
    if (r < a.rows) {
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
        if (jl >= j0 && jl < j1) {
#pragma unroll
          for (int f = 0; f < kNF; ++f) raw[jl][f] = ld_stream(x + r * kN + load_off(h, jl, f, lane));
        }
    }
  };
  if constexpr (!F32) load(blockIdx.x, 0, kPf);
  const float* xf = static_cast<const float*>(a.x);
  // fp32 input: stage 1 of own sub-row jl of row r, loaded here
  auto stage1_f32_sub = [&](int64_t r, int jl, float (&d)[kNF][2][4]) {
    uint4 r32[kNF][2];
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const float* p = xf + r * kN + load_off(h, jl, f, lane);
      r32[f][0] = ld_stream(p);
      r32[f][1] = ld_stream(p + 4);
    }
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      uint32_t th[4], tm[4], tl[4];
      split3_bf16(r32[f][0], r32[f][1], th, tm, tl);
      const uint4 mk = sign_masks(sb[jl], f);   // the signs flip every term
      const uint32_t m4[4] = {mk.x, mk.y, mk.z, mk.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) { th[k] ^= m4[k]; tm[k] ^= m4[k]; tl[k] ^= m4[k]; }
      bf16x8 ah, am, al;
      __builtin_memcpy(&ah, th, 16);
      __builtin_memcpy(&am, tm, 16);
      __builtin_memcpy(&al, tl, 16);
      const f32x4 p0 = stage1_f32(ah, am, al, hb[0]);
      const f32x4 p1 = stage1_f32(ah, am, al, hb[1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) { d[f][0][i] = p0[i]; d[f][1][i] = p1[i]; }
    }
  };

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const int64_t relem0 = row * kN;
    if constexpr (!F32) load(row, kPf, kOwn);
    // ---------------- stage 1: bits 0-4 ----------------
    // A first pass only takes the maximum: the split scale must exist before the first split,
    // and holding all 96 stage-1 values until then would leave room for one wave per SIMD.
    // The signed inputs stay in raw, and each sub-row's stage 1 is recomputed just before its
    // split (24 more matrix-core operations per row, on a unit with time to spare).
    float m1 = 0.0f;
    if constexpr (F32) {
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl) {
        float d[kNF][2][4];
        stage1_f32_sub(row, jl, d);
#pragma unroll
        for (int f = 0; f < kNF; ++f)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) m1 = fmaxf(m1, fabsf(d[f][t][i]));
      }
    } else {
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl)
#pragma unroll
        for (int f = 0; f < kNF; ++f) {
          uint4& r = raw[jl][f];
          const uint4 mk = sign_masks(sb[jl], f);
          r.x ^= mk.x; r.y ^= mk.y; r.z ^= mk.z; r.w ^= mk.w;
          const f32x4 p0 = stage1<H16>(r, hb[0]);
          const f32x4 p1 = stage1<H16>(r, hb[1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) m1 = fmaxf(m1, fmaxf(fabsf(p0[i]), fabsf(p1[i])));
        }
    }
    m1 = group_max(m1, 64);
    if (lane == 0) sh.m1[h] = m1;
    __syncthreads();   // every wave's maximum is in; the previous row's exchange reads are done
    m1 = fmaxf(fmaxf(sh.m1[0], sh.m1[1]), fmaxf(sh.m1[2], sh.m1[3]));
    float S, invS;
    split_scale(__float_as_uint(m1), S, invS);

    // w[j1][t][i2]: the twelve sub-rows at this wave's quarter, element 2048 j1 + 512 h + 8 lc + t + 2 i2
    float w[kSub][2][4];
#pragma unroll
    for (int jl = 0; jl < kOwn; ++jl) {
      float d1[kNF][2][4];   // [f][t][i]: stage 1 of this sub-row again
      if constexpr (F32) {
        stage1_f32_sub(row, jl, d1);
      } else {
#pragma unroll
        for (int f = 0; f < kNF; ++f) {
          const f32x4 p0 = stage1<H16>(raw[jl][f], hb[0]);
          const f32x4 p1 = stage1<H16>(raw[jl][f], hb[1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) { d1[f][0][i] = p0[i]; d1[f][1][i] = p1[i]; }
        }
      }
      // ---------------- stage 2: bits 5-9 of each 1024-half ----------------
      // d2[hf][t][t2][i2]: element 1024 hf + 512 t2 + 8 lc + t + 2 i2 of the sub-row
      float d2[2][2][2][4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float ys[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) ys[e] = d1[2 * hf + (e >> 2)][t][e & 3];
          uint32_t hw[4], lw[4];
          split8<true>(ys, S, hw, lw);   // ys are fresh matrix-core results
          f16x8 ah, al;
          __builtin_memcpy(&ah, hw, 16);
          __builtin_memcpy(&al, lw, 16);
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, hc[t2], z, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, hc[t2], acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) d2[hf][t][t2][i] = acc[i];
          }
        }
      // ---------------- bit 10, then hand the quarters out ----------------
      // quarter q = 2 hf' + t2 (hf' = output bit 10): y[q][t][i2]
      float y[4][2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = d2[0][t][t2][i], hi = d2[1][t][t2][i];
            y[t2][t][i] = lo + hi;
            y[2 + t2][t][i] = lo - hi;
          }
      // quarter q goes to wave q, d = (h - q) mod 4 behind this one: d = 1, 2 to LDS now; d = 3
      // waits in the registers of sub-row jl of wave h + 3, which the second exchange fills
#pragma unroll
      for (int q = 0; q < kW; ++q) {
        const int d = (h - q) & 3;
        if (d == 0 || d == 3) {
          const int j1 = d == 0 ? kOwn * h + jl : kOwn * ((h + 3) & 3) + jl;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) w[j1][t][i] = y[q][t][i];
        } else {
          sh.xb[d - 1][q][jl][0][lane] = make_float4(y[q][0][0], y[q][1][0], y[q][0][1], y[q][1][1]);
          sh.xb[d - 1][q][jl][1][lane] = make_float4(y[q][0][2], y[q][1][2], y[q][0][3], y[q][1][3]);
        }
      }
    }
    // the next row's loads go out once stage 1's values are consumed (registers allow no
    // earlier start) and run during the exchange, the order-12 factor and the epilogue
    if constexpr (!F32) load(row + gridDim.x, 0, kPf);
    auto take = [&](int slot, int j1, int jl) {
      const float4 u = sh.xb[slot][h][jl][0][lane];
      const float4 v = sh.xb[slot][h][jl][1][lane];
      w[j1][0][0] = u.x; w[j1][1][0] = u.y; w[j1][0][1] = u.z; w[j1][1][1] = u.w;
      w[j1][0][2] = v.x; w[j1][1][2] = v.y; w[j1][0][3] = v.z; w[j1][1][3] = v.w;
    };
    __syncthreads();   // the first exchange is in LDS
#pragma unroll
    for (int d = 1; d <= 2; ++d)
#pragma unroll
      for (int jl = 0; jl < kOwn; ++jl) take(d - 1, kOwn * ((h + d) & 3) + jl, jl);
    __syncthreads();   // every wave has read the first exchange
#pragma unroll
    for (int jl = 0; jl < kOwn; ++jl) {
      const int j1 = kOwn * ((h + 3) & 3) + jl;   // holds the quarter for wave h + 1
      sh.xb[0][(h + 1) & 3][jl][0][lane] = make_float4(w[j1][0][0], w[j1][1][0], w[j1][0][1], w[j1][1][1]);
      sh.xb[0][(h + 1) & 3][jl][1][lane] = make_float4(w[j1][0][2], w[j1][1][2], w[j1][0][3], w[j1][1][3]);
    }
    __syncthreads();   // the second exchange is in LDS
#pragma unroll
    for (int jl = 0; jl < kOwn; ++jl) take(0, kOwn * ((h + 3) & 3) + jl, jl);

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

    // chunk q = j1: elements 2048 q + 512 h + 8 lc + r
    auto val = [&](int q, int r) -> float { return w[q][r & 1][r >> 1]; };
    auto cbase = [&](int q) -> int { return kM * q + 512 * h; };

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
    } else if constexpr (BIG > 0) {
      fast24_big_groups<BIG, H>(a, sh, row, relem0, invS, cnorm, lane, lc, val, cbase);
    } else {
      // per-token INT4: maximum of the whole row across the four waves (uniform branch)
      auto rowmax = [&](float m) -> float {
        m = group_max(m, 64);
        if (lane == 0) sh.rmax[h] = m;
        __syncthreads();
        return fmaxf(fmaxf(sh.rmax[0], sh.rmax[1]), fmaxf(sh.rmax[2], sh.rmax[3]));
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
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale),
                __float_as_uint(nvfp4_tensor_scale(
                    fmaxf(fmaxf(sh.rmax[0], sh.rmax[1]), fmaxf(sh.rmax[2], sh.rmax[3])) * cnorm)));
  }
}

// H16: fp16 input (stage 1 on the f16 matrix-core instruction).
// BIG > 0: INT4 groups of 2^(9 + BIG) elements (a separate instantiation).  F32: fp32 input.
template <int OP, bool H16 = false, int BIG = 0, bool F32 = false>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(2))) void fast24_kernel(KernelArgs a) {
  __shared__ Shared24 sh;
  const int lane = threadIdx.x & 63;
  const int h = threadIdx.x >> 6;
  // the lane's own sign bits (the same for every row); none set without signs
  uint32_t sb[kOwn];
#pragma unroll
  for (int jl = 0; jl < kOwn; ++jl) sb[jl] = pack_signs(a.signs, h, jl, lane);
  const bf16x8 hb[2] = {h32_operand<H16>(lane, 0), h32_operand<H16>(lane, 1)};
  const f16x8 hc[2] = {h32_stage2_operand(lane, 0), h32_stage2_operand(lane, 1)};

  float gts = 0.0f, inv6g = 0.0f;
  if constexpr (OP == OP_NVFP4) {
    gts = a.tensor_scale[0];
    inv6g = gts > 0.0f ? 1.0f / (6.0f * gts) : 0.0f;
  }
  int G = 0;   // log2 of the INT4 group (0: one group per row)
  if constexpr (OP == OP_INT4) G = a.group == kN ? 0 : __builtin_ctz((unsigned)a.group);
  if constexpr (OP == OP_NVFP4) G = 4;
  if constexpr (OP == OP_MXFP4) G = 5;
  switch (h) {
    case 0: fast24_rows<OP, 0, H16, BIG, F32>(a, sh, hb, hc, sb, lane, gts, inv6g, G); break;
    case 1: fast24_rows<OP, 1, H16, BIG, F32>(a, sh, hb, hc, sb, lane, gts, inv6g, G); break;
    case 2: fast24_rows<OP, 2, H16, BIG, F32>(a, sh, hb, hc, sb, lane, gts, inv6g, G); break;
    default: fast24_rows<OP, 3, H16, BIG, F32>(a, sh, hb, hc, sb, lane, gts, inv6g, G); break;
  }
}

template <int OP, int IN, int BIG>
hipError_t launch24k(const KernelArgs& a, hipStream_t s) {
  auto kern = fast24_kernel<OP, IN == RHTQ_IN_F16, BIG, IN == RHTQ_IN_F32>;
  static const int max_blocks = resident_blocks((const void*)kern, kT, 0);
  const int grid = (int)(a.rows < max_blocks ? a.rows : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kT), 0, s, a);
  return hipGetLastError();
}

template <int OP, int IN>
hipError_t launch24(const KernelArgs& a, hipStream_t s) {
  if (a.sign_period != kN) return hipErrorNotSupported;
  if constexpr (OP == OP_INT4) {
    if (a.group == 1024) return launch24k<OP, IN, 1>(a, s);
    if (a.group == 2048) return launch24k<OP, IN, 2>(a, s);
    if (a.group == 4096) return launch24k<OP, IN, 3>(a, s);
    if (a.group == 8192) return launch24k<OP, IN, 4>(a, s);
    if (!(a.group == kN || (a.group >= 16 && a.group <= 512))) return hipErrorNotSupported;
  }
  return launch24k<OP, IN, 0>(a, s);
}

template <int IN>
hipError_t launch24_op(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return launch24<OP_ROTATE, IN>(a, s);
    case OP_INT4: return launch24<OP_INT4, IN>(a, s);
    case OP_NVFP4: return launch24<OP_NVFP4, IN>(a, s);
    case OP_MXFP4: return launch24<OP_MXFP4, IN>(a, s);
    case OP_AMAX: return launch24<OP_AMAX, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_fast24(int op, const KernelArgs& a, hipStream_t s, bool f16in) {
  return f16in ? launch24_op<RHTQ_IN_F16>(op, a, s) : launch24_op<RHTQ_IN_BF16>(op, a, s);
}

hipError_t launch_fast24_f32(int op, const KernelArgs& a, hipStream_t s) {
  return launch24_op<RHTQ_IN_F32>(op, a, s);
}

}  // namespace rhtq
