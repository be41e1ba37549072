// Matrix-core kernel for bf16 rows of 8192 and 16384 elements, n = 4096 x 2^B with B = 1, 2.
//
// A workgroup of W = 2^B waves owns one row at a time (persistent grid).  Wave K holds the
// sub-row j = 4096 K + [0, 4096) and runs on it the in-wave transform of the one-wave 4096
// kernel: 16-byte loads in the MFMA A layout with the sign masks (kept in registers for the
// whole kernel) XORed onto the bf16 sign bits, index bits 0-4 on v_mfma_f32_16x16x32_bf16
// against a +-1 H32, bits 5-9 on v_mfma_f32_16x16x32_f16 with every value split into two f16
// terms under a power-of-two scale S, bits 10-11 as register butterflies.  Afterwards the lane
// holds, per 1024-group g (bits 10-11) and half t2 (bit 9), eight consecutive outputs.
//
// The index bits 12 .. 11 + B pair the waves through LDS, one bit per round.  In round r, wave K
// and wave K ^ 2^r each keep the groups whose bit 1 - r equals their own bit r, send the other
// half (32 values per lane) and take the partner's values for the kept groups.  Both sides go to
// the smaller of their split scales (a power of two, folded into the butterfly as an FMA).  After
// the last round wave K owns the groups g with bit 1 - r of g equal to bit r of K, for every
// value of bits 12 and up: eight chunks of 512 consecutive outputs in the register layout of the
// one-wave kernel, so the shared epilogue quantises and stores them.  Per-token INT4 takes the
// row maximum across the waves through LDS.
//
// QuaRot reviews, review 1 Summary: online Hadamard by the Walsh-Hadamard fast algorithm;
// review 2 Summary: random Hadamard transform then INT4; reviewer 2 follow-up: nearest rounding.
// NVFP4 methodology thread: E2M1 codes with E4M3 block scales.
#include <hip/hip_fp16.h>

#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_epilogue.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

constexpr int kSub = 4096;   // elements of one wave's sub-row
constexpr int kNF = 8;       // 512-element fragments per sub-row

template <int W>
struct WideShared {
  uint4 xch[W][8][64];   // [wave][quad][lane]: the half a wave sends in the current round
  float xs[W];           // [wave]: split scale S in the current round
  float rmax[W];         // [wave]: row maximum (per-token INT4) or running maximum (tensor amax)
  float gmax[16];        // INT4 groups of whole 1024-element groups: the maximum of each (16384 only)
};

// INT4 groups of 2^(9 + BIG) elements (BIG = 1 .. 4: 1024 .. 8192) in 16384-wide rows.  After the
// exchange rounds wave K holds the 1024-element groups j = 4 s + gfix (s = 0 .. 3, chunks 2 s and
// 2 s + 1), so a group of 1024 is the wave's own and larger ones span two or four waves: each
// wave reduces its 1024-groups over its lanes, they meet in LDS behind one barrier (as the
// per-token maximum does), and every wave takes the maxima of its groups from there.
template <int BIG, int K, typename ValF, typename BaseF>
__device__ __forceinline__ void wide_big_groups(const KernelArgs& a, WideShared<4>& sh, const int64_t row,
                                                const int64_t ebase, const float invS, const float cnorm,
                                                const int lane, const int lc, ValF val, BaseF cbase) {
  constexpr int gfix = ((K & 1) << 1) | ((K >> 1) & 1);
  constexpr int LG = BIG - 1;          // log2 of the group in 1024-element groups
  float m1k[4];                        // this wave's 1024-groups, true units
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    float m = 0.0f;
#pragma unroll
    for (int q = 2 * st; q < 2 * st + 2; ++q)
#pragma unroll
      for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
    m1k[st] = group_max(m, 64) * invS;
  }
  if constexpr (LG > 0) {
    if (lane == 0) {
#pragma unroll
      for (int st = 0; st < 4; ++st) sh.gmax[4 * st + gfix] = m1k[st];
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int j0 = ((4 * st + gfix) >> LG) << LG;   // the group's first 1024-group
      float m = sh.gmax[j0];
#pragma unroll
      for (int j = 1; j < (1 << LG); ++j) m = fmaxf(m, sh.gmax[j0 + j]);
      m1k[st] = m;
    }
  }
  float inv[8];
  bool clamp = false;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const Int4Scale sc = int4_scale(m1k[st], cnorm, a.scale_dtype);
    clamp |= sc.clamp;
    inv[2 * st] = inv[2 * st + 1] = sc.inv * invS;
    // the wave holding the group's first 1024-group stores its scale
    const int j = 4 * st + gfix;
    if (lane == 0 && (j & ((1 << LG) - 1)) == 0) store_int4_scale(a.scales, a.scale_dtype, row * (16 >> LG) + (j >> LG), sc.s);
  }
  int4_codes<8>(a.packed + (ebase >> 1), inv, clamp, lc, val, cbase);
}

// values: v[slot][t][t2][i].  Before round r a slot is (h << (2 - r)) | c: h holds index bits
// 12 .. 11 + r, c the group bits of g not yet split (bits 0 .. 1 - r of g).
using Slots = float[4][2][2][4];

// The butterfly of round RD on the kept slots: own values a (index bit 12 + RD = kb) and the
// partner's b (bit 1 - kb); OC: own values are in the common units, else the partner's are.
template <int K, int RD, int W, bool OC>
__device__ __forceinline__ void combine_round(Slots& v, float f, WideShared<W>& sh, int lane) {
  constexpr int P = K ^ (1 << RD), kb = (K >> RD) & 1, sb = 1 - RD;
  float nv[4][2][2][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (((s >> sb) & 1) != kb) continue;
    const int j = ((s >> (sb + 1)) << sb) | (s & ((1 << sb) - 1));   // the partner sent this slot as j
    const int h = s >> (2 - RD), cp = s & ((1 << sb) - 1);
    const int s0 = (h << sb) | cp, s1 = ((h | (1 << RD)) << sb) | cp;   // new index bit 12 + RD = 0, 1
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const uint4 rv = sh.xch[P][4 * j + 2 * t + t2][lane];
        const float bo[4] = {__uint_as_float(rv.x), __uint_as_float(rv.y), __uint_as_float(rv.z),
                             __uint_as_float(rv.w)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = v[s][t][t2][i], b = bo[i];
          // y0 = (bit 0) + (bit 1), y1 = (bit 0) - (bit 1), the rescaled side through the FMA
          if constexpr (OC) {
            nv[s0][t][t2][i] = __builtin_fmaf(b, f, a);
            nv[s1][t][t2][i] = kb == 0 ? __builtin_fmaf(-b, f, a) : __builtin_fmaf(b, f, -a);
          } else {
            nv[s0][t][t2][i] = __builtin_fmaf(a, f, b);
            nv[s1][t][t2][i] = kb == 0 ? __builtin_fmaf(a, f, -b) : __builtin_fmaf(-a, f, b);
          }
        }
      }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[s][t][t2][i] = nv[s][t][t2][i];
}

template <int K, int RD, int W>
__device__ __forceinline__ void exchange_round(Slots& v, float& S, float& invS, WideShared<W>& sh, int lane) {
  constexpr int P = K ^ (1 << RD);          // partner wave
  constexpr int kb = (K >> RD) & 1;         // this wave keeps the slots whose split bit is kb
  constexpr int sb = 1 - RD;                // split bit of the slot (group bit 1 - RD)
  __syncthreads();   // the partner has read what this wave sent in the previous round
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (((s >> sb) & 1) == kb) continue;
    const int j = ((s >> (sb + 1)) << sb) | (s & ((1 << sb) - 1));   // rank among the sent slots
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
        sh.xch[K][4 * j + 2 * t + t2][lane] =
            make_uint4(__float_as_uint(v[s][t][t2][0]), __float_as_uint(v[s][t][t2][1]),
                       __float_as_uint(v[s][t][t2][2]), __float_as_uint(v[s][t][t2][3]));
  }
  if (lane == 0) sh.xs[K] = S;
  __syncthreads();
  // common units: the smaller split scale, so neither side is scaled up
  const float So = sh.xs[P];
  const bool own_common = S <= So;
  const float f = own_common ? S * __builtin_amdgcn_rcpf(So) : So * invS;   // power of two <= 1
  if (!own_common) {
    S = So;
    invS = __builtin_amdgcn_rcpf(So);
  }
  // (a uniform branch: each side is written out so that the rescale is one FMA per output)
  if (own_common) combine_round<K, RD, W, true>(v, f, sh, lane);
  else combine_round<K, RD, W, false>(v, f, sh, lane);
}

// Rows of the workgroup as seen by wave K (a template parameter, so that every register array
// is indexed by constants).  All waves of the workgroup take the same rows and barriers.
// H16: fp16 input (stage 1 on the f16 matrix-core instruction).  F32: fp32 input, each value split
// into three exact bf16 terms for stage 1 (split3_bf16, stage1_f32).  BIG > 0: INT4 groups of
// 2^(9 + BIG) elements at 16384 (wide_big_groups; a separate instantiation).
template <int B, int OP, int K, bool H16, bool F32, int BIG>
__device__ __forceinline__ void wide_rows(const KernelArgs& a, WideShared<1 << B>& sh) {
  constexpr int W = 1 << B, N = kSub << B;
  const int lane = threadIdx.x & 63;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)N));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const float* xf = static_cast<const float*>(a.x);
  const int lcol = 32 * (lane & 15) + 8 * (lane >> 4);   // this lane's 8 elements within a fragment
  const int lc = (lane >> 4) | ((lane & 15) << 2);       // element bits 3-4 = lane >> 4, 5-8 = lane & 15
  const bf16x8 hb[2] = {h32_operand<H16>(lane, 0), h32_operand<H16>(lane, 1)};
  const f16x8 hc[2] = {h32_stage2_operand(lane, 0), h32_stage2_operand(lane, 1)};
  // bf16 sign-bit masks of the 8 elements this lane loads in each fragment of its sub-row, held
  // in registers for the whole kernel (every row has the same signs)
  uint4 smask[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    smask[f] = make_uint4(0, 0, 0, 0);
    if (a.signs) {
      const uint2 sv = *reinterpret_cast<const uint2*>(a.signs + kSub * K + 512 * f + lcol);
      smask[f].x = __builtin_amdgcn_perm(0u, sv.x, 0x010C000Cu) & 0x80008000u;
      smask[f].y = __builtin_amdgcn_perm(0u, sv.x, 0x030C020Cu) & 0x80008000u;
      smask[f].z = __builtin_amdgcn_perm(0u, sv.y, 0x010C000Cu) & 0x80008000u;
      smask[f].w = __builtin_amdgcn_perm(0u, sv.y, 0x030C020Cu) & 0x80008000u;
    }
  }
  float gts = 0.0f, inv6g = 0.0f;
  if constexpr (OP == OP_NVFP4) {
    gts = a.tensor_scale[0];
    inv6g = gts > 0.0f ? 1.0f / (6.0f * gts) : 0.0f;
  }
  int G = 0;   // log2 of the INT4 group (0: one group per row)
  if constexpr (OP == OP_INT4) G = a.group == N ? 0 : __builtin_ctz((unsigned)a.group);
  if constexpr (OP == OP_NVFP4) G = 4;
  if constexpr (OP == OP_MXFP4) G = 5;
  // the group g this wave owns for slot s after the last round: bit 1 - r of g is bit r of K
  // (r < B); the bits below come from the slot
  constexpr int gfix = B == 1 ? ((K & 1) << 1) : (((K & 1) << 1) | ((K >> 1) & 1));
  float run_max = 0.0f;

  for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
    uint4 raw[F32 ? 1 : kNF];
    uint4 raw32[F32 ? kNF : 1][2];
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      if constexpr (F32) {
        const float* p = xf + row * N + kSub * K + 512 * f + lcol;
        raw32[f][0] = ld_stream(p);
        raw32[f][1] = ld_stream(p + 4);
      } else {
        raw[f] = ld_stream(x + row * N + kSub * K + 512 * f + lcol);
      }
    }

    // ---------------- stage 1: bits 0-4 ----------------
    float d1[kNF][2][4];
#pragma unroll
    for (int f = 0; f < kNF; ++f) {
      const uint4 m = smask[f];
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4 p0, p1;
      if constexpr (F32) {
        // the signs flip every term: the same bf16-pair masks
        uint32_t th[4], tm[4], tl[4];
        split3_bf16(raw32[f][0], raw32[f][1], th, tm, tl);
        const uint32_t mk[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) { th[k] ^= mk[k]; tm[k] ^= mk[k]; tl[k] ^= mk[k]; }
        bf16x8 ah, am, al;
        __builtin_memcpy(&ah, th, 16);
        __builtin_memcpy(&am, tm, 16);
        __builtin_memcpy(&al, tl, 16);
        p0 = stage1_f32(ah, am, al, hb[0]);
        p1 = stage1_f32(ah, am, al, hb[1]);
      } else {
        uint4 r = raw[f];
        r.x ^= m.x; r.y ^= m.y; r.z ^= m.z; r.w ^= m.w;
        bf16x8 av;
        __builtin_memcpy(&av, &r, 16);
        p0 = stage1_mma<H16>(av, hb[0], z);
        p1 = stage1_mma<H16>(av, hb[1], z);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) { d1[f][0][i] = p0[i]; d1[f][1][i] = p1[i]; }
    }
    float m1 = 0.0f;
#pragma unroll
    for (int f = 0; f < kNF; ++f)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) m1 = fmaxf(m1, fabsf(d1[f][t][i]));
    m1 = group_max(m1, 64);
    float S, invS;
    split_scale(__float_as_uint(m1), S, invS);

    // ---------------- stage 2: bits 5-9; v[g][t][t2][i] = element t + 2 i + 8 lc + 512 t2 + 1024 g ----------------
    Slots v;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float ys[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ys[e] = d1[2 * g + (e >> 2)][t][e & 3];
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
          for (int i = 0; i < 4; ++i) v[g][t][t2][i] = acc[i];
        }
      }
    // bits 10 and 11: register butterflies over g
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if ((g & (1 << b)) == 0)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
              for (int i = 0; i < 4; ++i) bfly(v[g][t][t2][i], v[g | (1 << b)][t][t2][i]);

    // ---------------- bits 12 ..: across the waves ----------------
    exchange_round<K, 0, W>(v, S, invS, sh, lane);
    if constexpr (B == 2) exchange_round<K, 1, W>(v, S, invS, sh, lane);

    // chunk q = 2 s + t2 of slot s: h = s >> (2 - B) (bits 12 ..), g = gfix | (s & ((4 >> B) - 1))
    auto val = [&](int q, int r) -> float { return v[q >> 1][r & 1][q & 1][r >> 1]; };
    auto cbase = [](int q) -> int {
      const int s = q >> 1;
      return 512 * (q & 1) + 1024 * (gfix | (s & ((4 >> B) - 1))) + 4096 * (s >> (2 - B));
    };
    const int64_t ebase = row * N;

    if constexpr (OP == OP_AMAX) {
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
      run_max = fmaxf(run_max, m * invS);   // across lanes and waves at the end
    } else if constexpr (OP == OP_ROTATE) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float o[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) o[r] = (val(q, r) * invS) * cnorm;
        float* p = a.y + ebase + cbase(q) + 8 * lc;
        st_stream(p, o[0], o[1], o[2], o[3]);
        st_stream(p + 4, o[4], o[5], o[6], o[7]);
      }
    } else if constexpr (BIG > 0) {
      static_assert(B == 2 && OP == OP_INT4, "large groups: INT4 at 16384");
      wide_big_groups<BIG, K>(a, sh, row, ebase, invS, cnorm, lane, lc, val, cbase);
    } else {
      quant_epilogue<OP, 8>(a, row, ebase, G, invS, cnorm, gts, inv6g, lane, lane == 0 && K == 0, val, cbase,
                            [&](float m) {
                              const float wm = group_max(m, 64);
                              if (lane == 0) sh.rmax[K] = wm;
                              __syncthreads();
                              float rm = sh.rmax[0];
#pragma unroll
                              for (int w = 1; w < W; ++w) rm = fmaxf(rm, sh.rmax[w]);
                              return rm;
                            });
    }
  }

  if constexpr (OP == OP_AMAX) {
    run_max = group_max(run_max, 64);
    __syncthreads();   // rmax is free (the rows above used it only for per-token INT4)
    if (lane == 0) sh.rmax[K] = run_max;
    __syncthreads();
    if (K == 0 && lane == 0) {
      float rm = sh.rmax[0];
#pragma unroll
      for (int w = 1; w < W; ++w) rm = fmaxf(rm, sh.rmax[w]);
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale), __float_as_uint(nvfp4_tensor_scale(rm * cnorm)));
    }
  }
}

template <int B, int OP, bool H16 = false, bool F32 = false, int BIG = 0>
__global__ __launch_bounds__(64 << B) void fastw_kernel(KernelArgs a) {
  __shared__ WideShared<1 << B> sh;
  const int wave = threadIdx.x >> 6;
  if constexpr (B == 1) {
    if (wave == 0) wide_rows<B, OP, 0, H16, F32, BIG>(a, sh);
    else wide_rows<B, OP, 1, H16, F32, BIG>(a, sh);
  } else {
    switch (wave) {
      case 0: wide_rows<B, OP, 0, H16, F32, BIG>(a, sh); break;
      case 1: wide_rows<B, OP, 1, H16, F32, BIG>(a, sh); break;
      case 2: wide_rows<B, OP, 2, H16, F32, BIG>(a, sh); break;
      default: wide_rows<B, OP, 3, H16, F32, BIG>(a, sh); break;
    }
  }
}

template <int B, int OP, int IN, int BIG>
hipError_t launchwk(const KernelArgs& a, hipStream_t s) {
  auto kern = fastw_kernel<B, OP, IN == RHTQ_IN_F16, IN == RHTQ_IN_F32, BIG>;
  static const int max_blocks = resident_blocks((const void*)kern, 64 << B, 0);
  const int grid = (int)(a.rows < max_blocks ? a.rows : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 << B), 0, s, a);
  return hipGetLastError();
}

template <int B, int OP, int IN>
hipError_t launchw(const KernelArgs& a, hipStream_t s) {
  constexpr int N = kSub << B;
  if (a.sign_period != N) return hipErrorNotSupported;   // block-diagonal calls: the other kernels
  if (reinterpret_cast<uintptr_t>(a.x) & 15) return hipErrorNotSupported;
  if constexpr (OP == OP_INT4) {
    if constexpr (B == 2) {   // groups of 1024 .. 8192 (8192: the single-stage kernel takes them)
      if (a.group == 1024) return launchwk<B, OP, IN, 1>(a, s);
      if (a.group == 2048) return launchwk<B, OP, IN, 2>(a, s);
      if (a.group == 4096) return launchwk<B, OP, IN, 3>(a, s);
      if (a.group == 8192) return launchwk<B, OP, IN, 4>(a, s);
    }
    if (!(a.group == N || (a.group >= 16 && a.group <= 512))) return hipErrorNotSupported;
  }
  return launchwk<B, OP, IN, 0>(a, s);
}

template <int OP, int IN>
hipError_t dispatchw(const KernelArgs& a, hipStream_t s) {
  switch (a.n) {
    case 8192: return launchw<1, OP, IN>(a, s);
    case 16384: return launchw<2, OP, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}

template <int IN>
hipError_t dispatchw_op(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return dispatchw<OP_ROTATE, IN>(a, s);
    case OP_INT4: return dispatchw<OP_INT4, IN>(a, s);
    case OP_NVFP4: return dispatchw<OP_NVFP4, IN>(a, s);
    case OP_MXFP4: return dispatchw<OP_MXFP4, IN>(a, s);
    case OP_AMAX: return dispatchw<OP_AMAX, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_fastw(int op, const KernelArgs& a, hipStream_t s, bool f16in) {
  return f16in ? dispatchw_op<RHTQ_IN_F16>(op, a, s) : dispatchw_op<RHTQ_IN_BF16>(op, a, s);
}

hipError_t launch_fastw_f32(int op, const KernelArgs& a, hipStream_t s) {
  return a.n == 16384 ? dispatchw_op<RHTQ_IN_F32>(op, a, s) : hipErrorNotSupported;
}

}  // namespace rhtq
