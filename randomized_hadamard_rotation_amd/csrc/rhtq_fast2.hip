// Two-stage matrix-core kernels for bf16 rows of 1024, 2048 and 4096 elements.
//
// fast2_kernel: one wavefront owns one row at a time (persistent grid).  fast2p_kernel (below,
// 4096-wide rows at small row counts) splits each row over two waves.  Per row:
//
//  1. Coalesced 16-byte loads in the MFMA A layout (lane l loads elements
//     512 f + 32 (l & 15) + 8 (l >> 4) + e of fragment f); random signs by XOR of bf16
//     sign bits with masks kept in LDS.
//  2. Stage 1: index bits 0-4 on v_mfma_f32_16x16x32_bf16 against a +-1 H32 operand.
//     bf16 times +-1 is exact, so this is the first five butterfly stages in fp32.
//     The result of tile t, register i, holds element
//         t + 2 (l & 15) + 32 i + 128 (l >> 4) + 512 f.
//  3. Stage 2: index bits 5-9 on v_mfma_f32_16x16x32_f16.  The stage-1 registers are
//     already in the A layout of this product (row = element bits 1-4, k = bits 5-9
//     spread over the register index i, the lane bits 4-5 and the fragment bit 9), so no
//     data moves between lanes.  fp32 does not fit an f16 operand, so each value y is
//     split as y S = hi + lo (two f16 terms, S a power of two chosen from the row
//     maximum so that |y S| < 2^15) and both halves go through the same +-1 operand;
//     the two products accumulate in fp32.  The split keeps 22 significant bits, and
//     the row-relative error stays near fp32 rounding.
//  4. Bits 10 and up (2048, 4096) are register butterflies.  Each lane now holds eight
//     consecutive outputs (element bits 0-2 in registers) and the 64 lanes cover 512
//     consecutive elements, so codes and values are stored straight from registers.
//  5. Epilogue: group maxima within the lane, then across lanes by pairwise
//     v_permlane16/32_swap + max that also compacts the groups into fewer registers,
//     so the scale arithmetic runs once per group; INT4 codes by the
//     round-to-nearest-even magic-constant FMA, E2M1 by v_cvt_scalef32_pk_fp4_f32 with
//     unit scale; nibble packing and 4-byte stores, 256 contiguous bytes per wave store.
//
// QuaRot reviews, review 1 Summary: online Hadamard by the Walsh-Hadamard fast
// algorithm; review 2 Summary: random Hadamard transform then INT4; reviewer 2
// follow-up: nearest rounding.  NVFP4 methodology thread: E2M1 codes with E4M3 block
// scales.
#include <hip/hip_fp16.h>

#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_epilogue.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

constexpr int kWaves2 = 4;
constexpr int kThreads2 = 64 * kWaves2;

template <int LOGM>
struct Shape2 {
  static constexpr int N = 1 << LOGM;
  static constexpr int NF = N / 512;        // stage-1 fragments (element bits 9..)
  static constexpr int NG = NF / 2;         // stage-2 output groups (element bits 10..)
  static constexpr int LOG_NG = LOGM - 10;
  static constexpr int R = 2 * NG;          // 512-element chunks per row (t2, g)
};

template <int LOGM>
__device__ __forceinline__ void load_row(const uint16_t* x, int64_t row, int64_t rows, int lane, uint4* raw) {
  using S2 = Shape2<LOGM>;
  if (row < rows) {   // past the last row raw[] is left as is: it is never used
#pragma unroll
    for (int f = 0; f < S2::NF; ++f) raw[f] = ld_stream(x + row * S2::N + 512 * f + 32 * (lane & 15) + 8 * (lane >> 4));
  }
}

// Prefetch depth (rows whose loads are in flight ahead of the current one) and the minimum waves
// per SIMD asked of the register allocator, by width.  Measured at 16384-65536 rows (INT4, MXFP4,
// NVFP4): without prefetch the registers leave room for three or four waves per SIMD at 4096
// (five to eight at the narrower widths), and those waves hide the load latency better than a
// two-row prefetch at two waves per SIMD did.
template <int LOGM>
struct Tune2 {
  static constexpr int DEPTH = 0;
  static constexpr int WAVES = LOGM == 10 ? 4 : 3;
};

// H16: fp16 input (stage 1 on the f16 matrix-core instruction; everything else is the same).
template <int LOGM, int OP, int DEPTH, int WAVES, bool H16 = false>
__global__ __launch_bounds__(kThreads2) __attribute__((amdgpu_waves_per_eu(WAVES)))
void fast2_kernel(KernelArgs a) {
  using S2 = Shape2<LOGM>;
  constexpr int N = S2::N, NF = S2::NF, NG = S2::NG, R = S2::R;
  extern __shared__ uint4 sign_tab[];   // [sign period / N][NF][64]
  __shared__ float wmax[kWaves2];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)N));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const int64_t rstride = (int64_t)gridDim.x * kWaves2;
  int64_t row = (int64_t)blockIdx.x * kWaves2 + wave;

  // DEPTH rows of loads in flight per wave: raw (this row) and raw2 (the next one);
  // DEPTH 0 loads each row at the top of its own step and relies on occupancy
  uint4 raw[NF] = {}, raw2[NF] = {};
  if constexpr (DEPTH >= 1) load_row<LOGM>(x, row, a.rows, lane, raw);
  if constexpr (DEPTH == 2) load_row<LOGM>(x, row + rstride, a.rows, lane, raw2);

  // bf16 sign-bit masks in load order: entry (slice * NF + f) * 64 + lane covers the 8 elements
  // that lane loads for fragment f of a row whose index is slice modulo the rows per sign period
  // (one slice unless the rows are blocks of longer rows)
  const int slices = a.sign_period / N;
  for (int k = threadIdx.x; k < slices * NF * 64; k += kThreads2) {
    uint4 m = make_uint4(0, 0, 0, 0);
    if (a.signs) {
      const int kl = k & 63, kf = k >> 6;
      const uint2 sv = *reinterpret_cast<const uint2*>(a.signs + N * (kf / NF) + 512 * (kf % NF) + 32 * (kl & 15) +
                                                       8 * (kl >> 4));
      m.x = __builtin_amdgcn_perm(0u, sv.x, 0x010C000Cu) & 0x80008000u;
      m.y = __builtin_amdgcn_perm(0u, sv.x, 0x030C020Cu) & 0x80008000u;
      m.z = __builtin_amdgcn_perm(0u, sv.y, 0x010C000Cu) & 0x80008000u;
      m.w = __builtin_amdgcn_perm(0u, sv.y, 0x030C020Cu) & 0x80008000u;
    }
    sign_tab[k] = m;
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
  if constexpr (OP == OP_INT4) G = a.group == N ? 0 : __builtin_ctz((unsigned)a.group);
  if constexpr (OP == OP_NVFP4) G = 4;
  if constexpr (OP == OP_MXFP4) G = 5;
  float run_max = 0.0f;
  // lane chunk: element bits 3-4 = lane >> 4, bits 5-8 = lane & 15
  const int lc = (lane >> 4) | ((lane & 15) << 2);

  auto step = [&](const int64_t row, uint4 (&raw)[NF]) {
    if constexpr (DEPTH == 0) load_row<LOGM>(x, row, a.rows, lane, raw);
    // ---------------- stage 1 ----------------
    float d1[NF][2][4];
    const int slice = slices > 1 ? (int)(row % slices) : 0;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint4 m = sign_tab[(slice * NF + f) * 64 + lane];
      uint4 r = raw[f];
      r.x ^= m.x; r.y ^= m.y; r.z ^= m.z; r.w ^= m.w;
      bf16x8 av;
      __builtin_memcpy(&av, &r, 16);
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4 p0 = stage1_mma<H16>(av, hb[0], z);
      const f32x4 p1 = stage1_mma<H16>(av, hb[1], z);
#pragma unroll
      for (int i = 0; i < 4; ++i) { d1[f][0][i] = p0[i]; d1[f][1][i] = p1[i]; }
    }
    // raw[] is consumed: it now receives the row DEPTH steps ahead, whose loads run
    // during the work of this and the following rows
    if constexpr (DEPTH >= 1) load_row<LOGM>(x, row + DEPTH * rstride, a.rows, lane, raw);

    // ---------------- split scale ----------------
    float m1 = 0.0f;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) m1 = fmaxf(m1, fabsf(d1[f][t][i]));
    m1 = group_max(m1, 64);
    float S, invS;
    split_scale(__float_as_uint(m1), S, invS);

    // ---------------- stage 2 ----------------
    // d2[t][g][t2][i2] holds element t + 2 i2 + 8 lc + 512 t2 + 1024 g
    float d2[2][NG][2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
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
          for (int i = 0; i < 4; ++i) d2[t][g][t2][i] = acc[i];
        }
      }
    // bits 10..: register butterflies over g
#pragma unroll
    for (int b = 0; b < S2::LOG_NG; ++b)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        if ((g & (1 << b)) == 0)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
              for (int i = 0; i < 4; ++i) bfly(d2[t][g][t2][i], d2[t][g | (1 << b)][t2][i]);

    // chunk q = t2 + 2 g: 8 consecutive elements per lane, y8[r] = element 8 lc + r
    auto val = [&](int q, int r) -> float { return d2[r & 1][q >> 1][q & 1][r >> 1]; };

    if constexpr (OP == OP_AMAX) {
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
      run_max = fmaxf(run_max, m * invS);   // across lanes at the end
      return;
    }

    const int64_t ebase = row * N;   // first element of the row

    if constexpr (OP == OP_ROTATE) {
#pragma unroll
      for (int q = 0; q < R; ++q) {
        float o[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) o[r] = (val(q, r) * invS) * cnorm;
        float* p = a.y + ebase + 512 * q + 8 * lc;
        st_stream(p, o[0], o[1], o[2], o[3]);
        st_stream(p + 4, o[4], o[5], o[6], o[7]);
      }
      return;
    }

    if constexpr (OP == OP_INT4 || OP == OP_NVFP4 || OP == OP_MXFP4)
      quant_epilogue<OP, R>(a, row, ebase, G, invS, cnorm, gts, inv6g, lane, lane == 0, val,
                            [](int q) { return 512 * q; }, [](float m) { return group_max(m, 64); });
  };
  if constexpr (DEPTH <= 1) {
    for (; row < a.rows; row += rstride) step(row, raw);
  } else {
    for (; row < a.rows; row += 2 * rstride) {
      step(row, raw);
      if (row + rstride < a.rows) step(row + rstride, raw2);
    }
  }

  if constexpr (OP == OP_AMAX) {
    run_max = group_max(run_max, 64);
    if (lane == 0) wmax[wave] = run_max;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = wmax[0];
#pragma unroll
      for (int w = 1; w < kWaves2; ++w) m = fmaxf(m, wmax[w]);
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale), __float_as_uint(nvfp4_tensor_scale(m * cnorm)));
    }
  }
}

// ---------------------------------------------------------------------------
// Small row counts at n = 4096: two waves per row, one row per workgroup (the workgroup barrier
// of the exchange then waits for the row's own two waves only).  With one wave per
// row a SIMD holds only the few rows the call has and sits idle while they wait on their own
// dependency chains; splitting each row doubles the waves and halves each chain.
//
// Linear layout: wave h takes the row half j = 2048 h + [0, 2048) as four 512-element
// fragments, and lane l loads the 16 bytes 512 f + 8 l of fragment f, so every wave load and
// store covers contiguous bytes in lane order.  In the MFMA A layout (row = lane & 15,
// k = 8 (lane >> 4) + e) that puts element bits 3-6 in the row and bits {0, 1, 2, 7, 8} in k:
// stage 1 transforms those five bits, stage 2 (same operand tables) bits {3, 4, 5, 6, 9}, and
// afterwards lane l holds the eight consecutive outputs 8 l + [0, 8) of every 512-element
// chunk.  (Any assignment of index bits to the stages gives the same Sylvester transform: the
// transform is a product of independent butterflies, one per bit.)
//
// Order of work: the constant operands and the signs (L2 hits) go out first, then the row's
// four fragments; each fragment's stage 1 runs as soon as it lands, with its share of the
// split-scale maximum.  Bit 10 (the fragment pair) is folded into stage 2 on the matrix
// cores: the outputs with bit 10 = 0 are A0 B + A1 B and those with bit 10 = 1 are A0 B - A1 B,
// so the two products share the A0 B partial and the second uses the negated operand.
// Bit 11 pairs the halves: wave h keeps its partial sums for the output chunks with bit 10 = h,
// sends the others through LDS, and both sides go to the smaller of the two split scales
// (powers of two, exact).  Wave h then owns the output chunks 1024 (2 h' + h) + [0, 1024),
// h' = 0, 1.  Per-row INT4 takes the row maximum over both waves through LDS.  Pairs past the
// last row repeat the last row (identical bytes), so all pairs of a workgroup always pass the
// same barriers.
// ---------------------------------------------------------------------------
#ifndef RHTQ_PAIR_WAVES
#define RHTQ_PAIR_WAVES 4
#endif
#ifndef RHTQ_PAIR_RPW
#define RHTQ_PAIR_RPW 1
#endif
constexpr int kPairRows = RHTQ_PAIR_RPW;   // rows per workgroup (two waves each)

// Stands in for an absent sign vector (all +1: no sign bits), so the sign loads need no branch.
__device__ __align__(16) int8_t kNoSigns[4096];

struct PairShared {
  uint4 xch[2][4][64];   // [wave h][value quad][lane]
  float xs[2];           // [h]: split scale S
  float rmax[2];         // [h]: row maximum of the half (true units)
};

// Wave H's half of one row (H a template parameter so every register array is indexed by
// constants).  H16: fp16 input.
template <int OP, int H, bool SLICED, bool H16>
__device__ __forceinline__ void pair_row(const KernelArgs& a, PairShared& sh, int64_t row) {
  constexpr int N = 4096;
  const int lane = threadIdx.x & 63;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)N));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const int lcol = 8 * lane;   // this lane's 8 elements within a fragment

  // constant operands and signs first (L2 hits), then the row's fragments; the scheduling
  // barriers keep that order, so each fragment's wait covers only the loads ahead of it
  const bf16x8 hb[2] = {h32_operand<H16>(lane, 0), h32_operand<H16>(lane, 1)};
  const f16x8 hc[2] = {h32_stage2_operand(lane, 0), h32_stage2_operand(lane, 1)};
  const f16x8 hn[2] = {h32_stage2_operand_neg(lane, 0), h32_stage2_operand_neg(lane, 1)};
  // SLICED: the rows are blocks of longer rows, and the block's slice of the sign vector
  // depends on the row (a 64-bit remainder, kept out of the plain call's code)
  int slice = 0;
  if constexpr (SLICED) slice = (int)(row % (a.sign_period / N));
  const int8_t* sg = (a.signs ? a.signs + N * slice : kNoSigns) + 2048 * H + lcol;
  uint2 sv[4];
#pragma unroll
  for (int fl = 0; fl < 4; ++fl) sv[fl] = *reinterpret_cast<const uint2*>(sg + 512 * fl);
  __builtin_amdgcn_sched_barrier(0);
  uint4 raw[4];
#pragma unroll
  for (int fl = 0; fl < 4; ++fl) raw[fl] = ld_stream(x + row * N + 2048 * H + 512 * fl + lcol);
  __builtin_amdgcn_sched_barrier(0);
  int G = 0;
  if constexpr (OP == OP_INT4) G = a.group == N ? 0 : __builtin_ctz((unsigned)a.group);
  if constexpr (OP == OP_NVFP4) G = 4;
  if constexpr (OP == OP_MXFP4) G = 5;

  // ---------------- stage 1, fragment by fragment as the loads land ----------------
  // d1[f][t][i]: output column lane & 15 of tile t, row 4 (lane >> 4) + i
  float d1[4][2][4];
  float m1 = 0.0f;
#pragma unroll
  for (int fl = 0; fl < 4; ++fl) {
    uint4 r = raw[fl];
    // bf16 sign-bit masks of the lane's 8 elements: bit 15 / bit 31 of each pair from byte bit 7
    r.x ^= __builtin_amdgcn_perm(0u, sv[fl].x, 0x010C000Cu) & 0x80008000u;
    r.y ^= __builtin_amdgcn_perm(0u, sv[fl].x, 0x030C020Cu) & 0x80008000u;
    r.z ^= __builtin_amdgcn_perm(0u, sv[fl].y, 0x010C000Cu) & 0x80008000u;
    r.w ^= __builtin_amdgcn_perm(0u, sv[fl].y, 0x030C020Cu) & 0x80008000u;
    bf16x8 av;
    __builtin_memcpy(&av, &r, 16);
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4 p0 = stage1_mma<H16>(av, hb[0], z);
    const f32x4 p1 = stage1_mma<H16>(av, hb[1], z);
#pragma unroll
    for (int i = 0; i < 4; ++i) { d1[fl][0][i] = p0[i]; d1[fl][1][i] = p1[i]; }
    // the previous fragment's maximum while this one's products run
    if (fl > 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) m1 = fmaxf(m1, fabsf(d1[fl - 1][t][i]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) m1 = fmaxf(m1, fabsf(d1[3][t][i]));
  m1 = group_max(m1, 64);
  float S, invS;
  split_scale(__float_as_uint(m1), S, invS);

  // ---------------- stage 2 with bit 10 ----------------
  // d2[t][gl][t2][i2]: element t + 2 i2 + 8 lane + 512 t2 + 1024 gl of this half
  float d2[2][2][2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f16x8 ah[2], al[2];
#pragma unroll
    for (int gl = 0; gl < 2; ++gl) {
      float ys[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ys[e] = d1[2 * gl + (e >> 2)][t][e & 3];
      uint32_t hw[4], lw[4];
      split8(ys, S, hw, lw);
      __builtin_memcpy(&ah[gl], hw, 16);
      __builtin_memcpy(&al[gl], lw, 16);
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[0], hc[t2], z, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[0], hc[t2], p, 0, 0, 0);
      f32x4 q0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[1], hc[t2], p, 0, 0, 0);
      q0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[1], hc[t2], q0, 0, 0, 0);
      f32x4 q1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[1], hn[t2], p, 0, 0, 0);
      q1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[1], hn[t2], q1, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) { d2[t][0][t2][i] = q0[i]; d2[t][1][t2][i] = q1[i]; }
    }
  }

  // ---------------- bit 11: exchange halves ----------------
  // sent: the partial sums with bit-10 index 1 - H, as quads q = 2 t + t2
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* sv = d2[q >> 1][1 - H][q & 1];
    sh.xch[H][q][lane] = make_uint4(__float_as_uint(sv[0]), __float_as_uint(sv[1]), __float_as_uint(sv[2]),
                                    __float_as_uint(sv[3]));
  }
  if (lane == 0) sh.xs[H] = S;
  __syncthreads();   // (workgroup-wide: both pairs of the workgroup pass it together)
  // common units: the smaller of the two split scales (the half with the larger maximum), so
  // neither side is scaled up; only the side with the larger scale is rescaled
  const float So = sh.xs[1 - H];
  const bool own_common = S <= So;
  const float f = own_common ? S * __builtin_amdgcn_rcpf(So) : So * invS;   // power of two <= 1
  if (!own_common) invS = __builtin_amdgcn_rcpf(So);
  // y2[hp][t][t2][i]: output element t + 2 i + 8 lane + 512 t2 + 1024 (2 hp + H)
  float y2[2][2][2][4];
  float r16[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 rv = sh.xch[1 - H][q][lane];
    r16[q][0] = __uint_as_float(rv.x); r16[q][1] = __uint_as_float(rv.y);
    r16[q][2] = __uint_as_float(rv.z); r16[q][3] = __uint_as_float(rv.w);
  }
  // y[j] = (half 0) + (half 1) and y[j + 2048] = (half 0) - (half 1), with the rescale by the
  // power of two f folded into one FMA per output (the product is exact, so this equals the
  // multiply-then-add); a uniform branch picks which side is rescaled
  if (own_common) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float own = d2[q >> 1][H][q & 1][i], oth = r16[q][i];
        y2[0][q >> 1][q & 1][i] = __builtin_fmaf(oth, f, own);
        y2[1][q >> 1][q & 1][i] = H == 0 ? __builtin_fmaf(-oth, f, own) : __builtin_fmaf(oth, f, -own);
      }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float own = d2[q >> 1][H][q & 1][i], oth = r16[q][i];
        y2[0][q >> 1][q & 1][i] = __builtin_fmaf(own, f, oth);
        y2[1][q >> 1][q & 1][i] = H == 0 ? __builtin_fmaf(own, f, -oth) : __builtin_fmaf(-own, f, oth);
      }
  }

  auto val = [&](int q, int r) -> float { return y2[q >> 1][r & 1][q & 1][r >> 1]; };
  auto cbase = [](int q) { return 512 * (q & 1) + 2048 * (q >> 1) + 1024 * H; };
  const int64_t ebase = row * N;

  if constexpr (OP == OP_AMAX) {
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
    m = group_max(m * invS, 64);
    if (lane == 0) sh.rmax[H] = m;
    __syncthreads();
    if (lane == 0 && H == 0)   // one atomic per row (per pair)
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale),
                __float_as_uint(nvfp4_tensor_scale(fmaxf(sh.rmax[0], sh.rmax[1]) * cnorm)));
  } else if constexpr (OP == OP_ROTATE) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float o[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) o[r] = (val(q, r) * invS) * cnorm;
      float* p = a.y + ebase + cbase(q) + 8 * lane;
      st_stream(p, o[0], o[1], o[2], o[3]);
      st_stream(p + 4, o[4], o[5], o[6], o[7]);
    }
  } else {
    float gts = 0.0f, inv6g = 0.0f;
    if constexpr (OP == OP_NVFP4) {
      gts = a.tensor_scale[0];
      inv6g = gts > 0.0f ? 1.0f / (6.0f * gts) : 0.0f;
    }
    quant_epilogue_lin<OP, 4>(a, row, ebase, G, invS, cnorm, gts, inv6g, lane, lane == 0 && H == 0, val, cbase,
                          [&](float m) {
                            const float wm = group_max(m, 64);
                            if (lane == 0) sh.rmax[H] = wm;
                            __syncthreads();
                            return fmaxf(sh.rmax[0], sh.rmax[1]);
                          });
  }
}

template <int OP, bool SLICED, bool H16 = false>
__global__ __launch_bounds__(128 * kPairRows) __attribute__((amdgpu_waves_per_eu(RHTQ_PAIR_WAVES))) void fast2p_kernel(KernelArgs a) {
  __shared__ PairShared sh[kPairRows];
  const int wave = threadIdx.x >> 6, pair = wave >> 1;
  int64_t row = kPairRows * (int64_t)blockIdx.x + pair;
  if (row >= a.rows) row = a.rows - 1;   // past the end: repeat the last row (same bytes, same barriers)
  if (wave & 1) pair_row<OP, 1, SLICED, H16>(a, sh[pair], row);
  else pair_row<OP, 0, SLICED, H16>(a, sh[pair], row);
}

template <int OP, bool H16>
hipError_t launch2p(const KernelArgs& a, hipStream_t s) {
  if constexpr (OP == OP_INT4) {
    if (!(a.group == 4096 || (a.group >= 16 && a.group <= 512))) return hipErrorNotSupported;
  }
  if (a.rows > 0xFFFFFFFE) return hipErrorNotSupported;
  const dim3 grid((unsigned)((a.rows + kPairRows - 1) / kPairRows));
  if (a.sign_period == 4096) hipLaunchKernelGGL((fast2p_kernel<OP, false, H16>), grid, dim3(128 * kPairRows), 0, s, a);
  else hipLaunchKernelGGL((fast2p_kernel<OP, true, H16>), grid, dim3(128 * kPairRows), 0, s, a);
  return hipGetLastError();
}

template <int LOGM, int OP, bool H16>
hipError_t launch2(const KernelArgs& a, hipStream_t s) {
  using S2 = Shape2<LOGM>;
  if constexpr (OP == OP_INT4) {
    if (!(a.group == S2::N || (a.group >= 16 && a.group <= 512))) return hipErrorNotSupported;
  }
  auto kern = fast2_kernel<LOGM, OP, Tune2<LOGM>::DEPTH, Tune2<LOGM>::WAVES, H16>;
  static const int max_blocks = resident_blocks((const void*)kern, kThreads2, S2::NF * 64 * 16);
  const int64_t want = (a.rows + kWaves2 - 1) / kWaves2;
  const int grid = (int)(want < max_blocks ? want : max_blocks);
  const size_t lds = (size_t)(a.sign_period / S2::N) * S2::NF * 64 * 16;
  if (lds > 65536) return hipErrorNotSupported;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads2), lds, s, a);
  return hipGetLastError();
}

// Row counts up to this use two waves per 4096-wide row (RHTQ_PAIR_ROWS overrides; read once).
inline int64_t pair_rows_limit() {
  static const int64_t v = [] {
    const char* e = getenv("RHTQ_PAIR_ROWS");
    return e != nullptr ? (int64_t)atoll(e) : (int64_t)4096;
  }();
  return v;
}

template <int OP, bool H16>
hipError_t dispatch2(const KernelArgs& a, hipStream_t s) {
  switch (a.n) {
    case 1024: return launch2<10, OP, H16>(a, s);
    case 2048: return launch2<11, OP, H16>(a, s);
    case 4096:
      if (a.rows <= pair_rows_limit()) {
        const hipError_t e = launch2p<OP, H16>(a, s);
        if (e != hipErrorNotSupported) return e;
      }
      return launch2<12, OP, H16>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

namespace {
template <bool H16>
hipError_t dispatch2_op(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return dispatch2<OP_ROTATE, H16>(a, s);
    case OP_INT4: return dispatch2<OP_INT4, H16>(a, s);
    case OP_NVFP4: return dispatch2<OP_NVFP4, H16>(a, s);
    case OP_MXFP4: return dispatch2<OP_MXFP4, H16>(a, s);
    case OP_AMAX: return dispatch2<OP_AMAX, H16>(a, s);
    default: return hipErrorNotSupported;
  }
}
}  // namespace

hipError_t launch_fast2(int op, const KernelArgs& a, hipStream_t s, bool f16in) {
  return f16in ? dispatch2_op<true>(op, a, s) : dispatch2_op<false>(op, a, s);
}

}  // namespace rhtq
