// Register-resident kernels for bf16 input on gfx950.
//
// One wavefront owns one row (rows of >= 512 elements) or one 512-element block of
// consecutive rows (16- to 256-wide rows) at a time and loops over rows
// (persistent grid).  Per row:
//
//  1. Coalesced 16-byte loads in the MFMA A-operand layout: lane l loads the 8
//     elements j = 512 f + 32 (l & 15) + 8 (l >> 4) + e of fragment f, so one load
//     instruction covers 512 consecutive elements.  The random signs are applied by
//     XOR-ing bf16 sign bits with masks kept in LDS.
//  2. The first five index bits (0..4) are transformed by v_mfma_f32_16x16x32_bf16
//     against a constant +-1 Sylvester H32 operand (for 16-wide rows the block-diagonal
//     I2 (x) H16, bit 4 being a row bit).  The input is exact bf16 and the
//     matrix is +-1, so every product is exact and the sums are fp32 accumulations,
//     the same arithmetic as the first five butterfly stages.
//  3. The remaining bits run as fp32 butterflies in registers: bits 5-6 and the
//     fragment bits (9..) are register indices; bits 7-8 sit in lane bits 4-5 and are
//     brought into registers with v_permlane16_swap / v_permlane32_swap.
//  4. n = 12 m: the order-12 Williamson factor is applied in registers across the
//     twelve sub-rows (KronQ issue #2, Model Details: 12288 = 12 x 1024).
//  5. Epilogue: 512/1024-element chunks go through a per-wave LDS buffer so that each
//     lane holds 8 or 16 consecutive elements; then group maxima (DPP), scales,
//     quantisation (INT4 by the round-to-nearest-even magic-constant FMA; E2M1 by
//     v_cvt_scalef32_pk_fp4_f32 with unit scale), nibble packing and 8-byte stores.
//
// QuaRot reviews, review 1 Summary: the online Hadamard uses the Walsh-Hadamard fast
// algorithm; review 2 Summary: random Hadamard transform then INT4; reviewer 2
// follow-up: nearest rounding.  NVFP4 methodology thread: E2M1 + E4M3 block scales.
#include <hip/hip_fp16.h>

#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int F, int LOGM>
struct Shape {
  static constexpr int M = 1 << LOGM;                  // power-of-two factor
  static constexpr int N = F * M;                      // row width
  static constexpr int UNIT = N >= 512 ? N : 512;      // elements per wave iteration
  static constexpr int RPU = UNIT / N;                 // rows per unit (1, 2, 4, 8, 16 or 32)
  static constexpr int NF = UNIT / 512;                // MFMA fragments per unit
  // fragments per power-of-two sub-row (for 12 x 256 a sub-row is half a fragment: 1, no
  // fragment-bit butterflies)
  static constexpr int FPJ = (F == 12) ? (M >= 512 ? M / 512 : 1) : NF;
  static constexpr int LOG_FPJ = FPJ == 1 ? 0 : (FPJ == 2 ? 1 : (FPJ == 4 ? 2 : (FPJ == 8 ? 3 : 4)));
  static constexpr int CHUNK = M >= 1024 ? 1024 : 512; // epilogue transpose unit
  static constexpr int NCH = UNIT / CHUNK;
  static constexpr int FPC = CHUNK / 512;              // fragments per chunk
  static constexpr int V = CHUNK / 64;                 // consecutive elements per lane after transpose
  static constexpr int TBUF = CHUNK + CHUNK / 8;       // padded chunk buffer (floats)
  static constexpr bool BIT5 = (F == 12) || LOGM >= 6; // bit 5 inside the power-of-two sub-row
  static constexpr bool BIT6 = (F == 12) || LOGM >= 7; // bit 6 inside the power-of-two sub-row
  static constexpr bool BIT7 = (F == 12) || LOGM >= 8; // bit 7 inside the power-of-two sub-row
  static constexpr bool BIT8 = LOGM >= 9;              // bit 8 inside the power-of-two sub-row
  // 12 x 256: bit 8 is the low bit of the order-12 index j1, so it is brought into registers
  // without a butterfly and the order-12 factor runs after the lane swaps
  static constexpr bool H12_LATE = (F == 12) && LOGM == 8;
  static constexpr bool SWAP8 = BIT8 || H12_LATE;
  // loads of the next unit overlap this unit's work when the registers allow it
  static constexpr bool PREFETCH = NF <= 8;
};

// padded LDS index of a chunk-local element: 4 extra floats after every 32, so the
// 8-byte pair stores and the 16-byte reads of 8 or 16 consecutive floats per lane touch
// distinct banks
__device__ __forceinline__ int tpad(int j) { return j + ((j >> 5) << 2); }

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Issue the 16-byte loads of unit u (fragment f at element 512 f + 32 (l & 15) + 8 (l >> 4));
// elements past the last row read as zero.
template <typename S>
__device__ __forceinline__ void load_unit(const uint16_t* x, int64_t u, int64_t units, int64_t rows,
                                          int lane, uint4* raw) {
  const int64_t valid = (rows - u * S::RPU) * S::N;
#pragma unroll
  for (int f = 0; f < S::NF; ++f) {
    const int off = 512 * f + 32 * (lane & 15) + 8 * (lane >> 4);
    raw[f] = make_uint4(0, 0, 0, 0);
    if (u < units && (S::RPU == 1 || off < valid))
      raw[f] = ld_stream(x + u * S::UNIT + off);
  }
}

// fp32 input: the same eight elements per lane and fragment as two 16-byte loads (elements
// 0-3 and 4-7 of the lane's run).
template <typename S>
__device__ __forceinline__ void load_unit_f32(const float* x, int64_t u, int64_t units, int64_t rows, int lane,
                                              uint4 (*raw)[2]) {
  const int64_t valid = (rows - u * S::RPU) * S::N;
#pragma unroll
  for (int f = 0; f < S::NF; ++f) {
    const int off = 512 * f + 32 * (lane & 15) + 8 * (lane >> 4);
    raw[f][0] = make_uint4(0, 0, 0, 0);
    raw[f][1] = make_uint4(0, 0, 0, 0);
    if (u < units && (S::RPU == 1 || off < valid)) {
      raw[f][0] = ld_stream(x + u * S::UNIT + off);
      raw[f][1] = ld_stream(x + u * S::UNIT + off + 4);
    }
  }
}

// Units of the sign table: lcm(UNIT, sign period) / UNIT (UNIT is a power of two).
template <typename S>
__host__ __device__ inline int sign_slices(int period) {
  int g = S::UNIT;
  while (period % g) g >>= 1;   // gcd(period, UNIT)
  return period / g;            // lcm / UNIT = period / gcd
}

// CG: INT4 groups of two or more whole chunks, short of the row (a separate instantiation, so the
// common kernels carry no code or registers for them).  F32: fp32 input, split into three exact
// bf16 terms for the stage-1 products (three MFMAs accumulating where bf16 input takes one), no
// prefetch; everything after stage 1 is the bf16 kernel's.  H16: fp16 input, the same loads and
// sign masks with stage 1 on the f16 matrix-core instruction.
template <int F, int LOGM, int OP, bool CG = false, bool F32 = false, bool H16 = false>
__global__ __launch_bounds__(kThreads) void fast_kernel(KernelArgs a) {
  using S = Shape<F, LOGM>;
  extern __shared__ uint32_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float* tbuf = reinterpret_cast<float*>(smem + sign_slices<S>(a.sign_period) * S::NF * 256) + wave * S::TBUF;

  const float cnorm = (float)(1.0 / __builtin_sqrt((double)S::N));
  const int64_t units = (a.rows + S::RPU - 1) / S::RPU;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const int64_t ustride = (int64_t)gridDim.x * kWaves;
  int64_t u = (int64_t)blockIdx.x * kWaves + wave;

  // The first unit's loads go out before the table setup so both latencies overlap.
  constexpr bool PREFETCH = S::PREFETCH && !F32;
  uint4 raw[F32 ? 1 : S::NF];
  uint4 raw32[F32 ? S::NF : 1][2];
  const float* xf = static_cast<const float*>(a.x);
  if constexpr (F32) load_unit_f32<S>(xf, u, units, a.rows, lane, raw32);
  else load_unit<S>(x, u, units, a.rows, lane, raw);

  // bf16 sign-bit masks in load order: entry (slice * NF + f) * 64 + lane holds the four mask
  // dwords (bit 15 / bit 31 of each bf16 pair) of the 8 elements that lane loads for fragment f of
  // a unit starting at element slice * UNIT modulo lcm(UNIT, sign period): one slice unless the rows
  // are blocks of longer rows.
  uint4* sign_tab = reinterpret_cast<uint4*>(smem);
  const int slices = sign_slices<S>(a.sign_period);
  for (int k = threadIdx.x; k < slices * S::NF * 64; k += kThreads) {
    uint4 m = make_uint4(0, 0, 0, 0);
    if (a.signs) {
      const int kl = k & 63, kf = k >> 6;   // kf = slice * NF + f
      const int col = (S::UNIT * (kf / S::NF) + 512 * (kf % S::NF) + 32 * (kl & 15) + 8 * (kl >> 4)) % a.sign_period;
      const uint2 sv = *reinterpret_cast<const uint2*>(a.signs + col);
      m.x = __builtin_amdgcn_perm(0u, sv.x, 0x010C000Cu) & 0x80008000u;
      m.y = __builtin_amdgcn_perm(0u, sv.x, 0x030C020Cu) & 0x80008000u;
      m.z = __builtin_amdgcn_perm(0u, sv.y, 0x010C000Cu) & 0x80008000u;
      m.w = __builtin_amdgcn_perm(0u, sv.y, 0x030C020Cu) & 0x80008000u;
    }
    sign_tab[k] = m;
  }
  // stage-1 operand: H32 over element bits 0-4, or I2 (x) H16 for 16-wide rows (bit 4 = row)
  const bf16x8 hb[2] = {LOGM == 4 ? h16_operand<H16>(lane, 0) : h32_operand<H16>(lane, 0),
                        LOGM == 4 ? h16_operand<H16>(lane, 1) : h32_operand<H16>(lane, 1)};
  __syncthreads();
  float run_max = 0.0f;
  float gts = 0.0f, inv6g = 0.0f;
  if constexpr (OP == OP_NVFP4) {
    gts = a.tensor_scale[0];
    inv6g = gts > 0.0f ? 1.0f / (6.0f * gts) : 0.0f;
  }

  for (; u < units; u += ustride) {
    if constexpr (!PREFETCH) {
      if (u != (int64_t)blockIdx.x * kWaves + wave) {
        if constexpr (F32) load_unit_f32<S>(xf, u, units, a.rows, lane, raw32);
        else load_unit<S>(x, u, units, a.rows, lane, raw);
      }
    }
    const int64_t ubase = u * S::UNIT;                 // element index of the unit start
    const int slice = slices > 1 ? (int)((ubase % ((int64_t)slices * S::UNIT)) / S::UNIT) : 0;
    const int64_t valid = (a.rows - u * S::RPU) * S::N;  // elements of the unit that exist (may exceed UNIT)

    // ---------------- sign, MFMA ----------------
    float v[S::NF][2][4];
#pragma unroll
    for (int f = 0; f < S::NF; ++f) {
      const uint4 m = sign_tab[(slice * S::NF + f) * 64 + lane];
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4 d0, d1;
      if constexpr (F32) {
        // the sign flips every term's sign bit: the same bf16-pair masks as for bf16 input
        uint32_t th[4], tm[4], tl[4];
        split3_bf16(raw32[f][0], raw32[f][1], th, tm, tl);
        const uint32_t mk[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) { th[k] ^= mk[k]; tm[k] ^= mk[k]; tl[k] ^= mk[k]; }
        bf16x8 ah, am, al;
        __builtin_memcpy(&ah, th, 16);
        __builtin_memcpy(&am, tm, 16);
        __builtin_memcpy(&al, tl, 16);
        d0 = stage1_f32(ah, am, al, hb[0]);
        d1 = stage1_f32(ah, am, al, hb[1]);
      } else {
        uint4 r = raw[f];
        r.x ^= m.x; r.y ^= m.y; r.z ^= m.z; r.w ^= m.w;
        bf16x8 av;
        __builtin_memcpy(&av, &r, 16);
        d0 = stage1_mma<H16>(av, hb[0], z);
        d1 = stage1_mma<H16>(av, hb[1], z);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[f][0][i] = d0[i]; v[f][1][i] = d1[i]; }
    }
    // raw[] is consumed: its registers now receive the next unit, whose loads run while
    // this unit's butterflies and epilogue execute
    if constexpr (PREFETCH) load_unit<S>(x, u + ustride, units, a.rows, lane, raw);

    // ---------------- butterflies on register bits ----------------
    // bits 5, 6: register index i (bit 5 = i & 1, bit 6 = i >> 1), where they lie inside the row
#pragma unroll
    for (int f = 0; f < S::NF; ++f)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (S::BIT5) {
          bfly(v[f][t][0], v[f][t][1]);
          bfly(v[f][t][2], v[f][t][3]);
        }
        if constexpr (S::BIT6) {
          bfly(v[f][t][0], v[f][t][2]);
          bfly(v[f][t][1], v[f][t][3]);
        }
      }
    // bits 9.. inside each power-of-two sub-row: fragment index
#pragma unroll
    for (int b = 0; b < S::LOG_FPJ; ++b)
#pragma unroll
      for (int f = 0; f < S::NF; ++f)
        if (((f % S::FPJ) & (1 << b)) == 0)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) bfly(v[f][t][i], v[f + (1 << b)][t][i]);
    // order-12 factor across the twelve sub-rows (whole fragments each)
    if constexpr (F == 12 && !S::H12_LATE) {
#pragma unroll
      for (int fl = 0; fl < S::FPJ; ++fl)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float w[12];
#pragma unroll
            for (int j1 = 0; j1 < 12; ++j1) w[j1] = v[j1 * S::FPJ + fl][t][i];
            h12_forward(w);
#pragma unroll
            for (int j1 = 0; j1 < 12; ++j1) v[j1 * S::FPJ + fl][t][i] = w[j1];
          }
    }
    // bit 7 (lane bit 4) and bit 8 (lane bit 5): exchange with register bits 5 / 6
    if constexpr (S::BIT7) {
#pragma unroll
      for (int f = 0; f < S::NF; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[f][t][i]),
                                                      __float_as_uint(v[f][t][i + 1]), false, false);
            v[f][t][i] = __uint_as_float(p[0]);
            v[f][t][i + 1] = __uint_as_float(p[1]);
            bfly(v[f][t][i], v[f][t][i + 1]);
          }
    }
    if constexpr (S::SWAP8) {
#pragma unroll
      for (int f = 0; f < S::NF; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[f][t][i]),
                                                      __float_as_uint(v[f][t][i + 2]), false, false);
            v[f][t][i] = __uint_as_float(p[0]);
            v[f][t][i + 2] = __uint_as_float(p[1]);
            if constexpr (S::BIT8) bfly(v[f][t][i], v[f][t][i + 2]);
          }
    }
    // 12 x 256: j = 256 j1 + j2 with j1 = 2 f + (element bit 8 = register bit i >> 1)
    if constexpr (S::H12_LATE) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i0 = 0; i0 < 2; ++i0) {
          float w[12];
#pragma unroll
          for (int j1 = 0; j1 < 12; ++j1) w[j1] = v[j1 >> 1][t][i0 | ((j1 & 1) << 1)];
          h12_forward(w);
#pragma unroll
          for (int j1 = 0; j1 < 12; ++j1) v[j1 >> 1][t][i0 | ((j1 & 1) << 1)] = w[j1];
        }
    }
    // Element held by (f, t, i) at this lane, within the unit (rows >= 512 wide):
    //   j = 512 f + 128 i + 32 (lane >> 4) + 2 (lane & 15) + t
    // 256-wide rows (bit 8 = row):  j = 256 (lane >> 5) + 128 (i & 1) + 64 (i >> 1) + 32 ((lane >> 4) & 1) + 2 (lane & 15) + t
    // 128-wide rows (bits 7-8 = row): j = 128 (lane >> 4) + 32 i + 2 (lane & 15) + t
    //   (the same for 64-, 32- and 16-wide rows, whose bits 6.., 5.. and 4.. select the row)

    if constexpr (OP == OP_AMAX) {
#pragma unroll
      for (int f = 0; f < S::NF; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) run_max = fmaxf(run_max, fabsf(v[f][t][i]));
      continue;
    }

    // per-token groups wider than a chunk: row maximum now (whole unit is one row)
    const bool row_group = (OP == OP_INT4) && (a.group == S::N) && (S::N > S::CHUNK);
    Int4Scale row_sc{0.0f, 0.0f, false};
    if (row_group) {
      float row_amax = 0.0f;
#pragma unroll
      for (int f = 0; f < S::NF; ++f)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) row_amax = fmaxf(row_amax, fabsf(v[f][t][i]));
      row_sc = int4_scale(group_max(row_amax, 64), cnorm, a.scale_dtype);
    }
    // groups of two or more whole chunks, short of the row (a power of two: 2048 at 4096,
    // 2048 and 4096 at 8192, 1024 at 3072, 1024 and 2048 at 6144): each chunk's maximum over the
    // wave now, then the maximum over the chunks of its group; chunk c holds fragments
    // FPC c .. FPC c + FPC - 1, i.e. elements CHUNK c + [0, CHUNK)
    constexpr bool chunk_groups = CG && (OP == OP_INT4);
    Int4Scale chunk_sc[S::NCH];
    if constexpr (chunk_groups) {
      float cm[S::NCH];
#pragma unroll
      for (int c = 0; c < S::NCH; ++c) {
        float m = 0.0f;
#pragma unroll
        for (int fc = 0; fc < S::FPC; ++fc)
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(v[S::FPC * c + fc][t][i]));
        cm[c] = group_max(m, 64);
      }
      const int cpg = a.group / S::CHUNK;   // chunks per group
#pragma unroll
      for (int c = 0; c < S::NCH; ++c) {
        float gm = 0.0f;
#pragma unroll
        for (int c2 = 0; c2 < S::NCH; ++c2)
          if (c2 / cpg == c / cpg) gm = fmaxf(gm, cm[c2]);
        chunk_sc[c] = int4_scale(gm, cnorm, a.scale_dtype);
      }
    }

    // ---------------- epilogue, one chunk at a time ----------------
#pragma unroll
    for (int c = 0; c < S::NCH; ++c) {
      // registers of chunk c -> LDS in element order
#pragma unroll
      for (int fc = 0; fc < S::FPC; ++fc) {
        const int f = c * S::FPC + fc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int jl;
          if constexpr (S::N >= 512 || F == 12)
            jl = 512 * fc + 128 * i + 32 * (lane >> 4) + 2 * (lane & 15);
          else if constexpr (S::N == 256)
            jl = 256 * (lane >> 5) + 128 * (i & 1) + 64 * (i >> 1) + 32 * ((lane >> 4) & 1) + 2 * (lane & 15);
          else
            jl = 128 * (lane >> 4) + 32 * i + 2 * (lane & 15);
          *reinterpret_cast<float2*>(tbuf + tpad(jl)) = make_float2(v[f][0][i], v[f][1][i]);
        }
      }
      lds_fence();
      float y[S::V];
#pragma unroll
      for (int q = 0; q < S::V / 4; ++q) {
        const float4 r = *reinterpret_cast<const float4*>(tbuf + tpad(S::V * lane + 4 * q));
        y[4 * q + 0] = r.x; y[4 * q + 1] = r.y; y[4 * q + 2] = r.z; y[4 * q + 3] = r.w;
      }
      // LDS requests of a wave complete in order: the next chunk's stores cannot overtake
      // these loads, so only compiler ordering is needed here.
      asm volatile("" ::: "memory");

      const int64_t g0 = ubase + (int64_t)c * S::CHUNK + S::V * lane;   // first element of this lane
      const bool live = (S::RPU == 1) || ((int64_t)c * S::CHUNK + S::V * lane < valid);

      if constexpr (OP == OP_ROTATE) {
        if (live) {
#pragma unroll
          for (int q = 0; q < S::V / 4; ++q)
            st_stream(a.y + g0 + 4 * q, y[4 * q] * cnorm, y[4 * q + 1] * cnorm, y[4 * q + 2] * cnorm,
                      y[4 * q + 3] * cnorm);
        }
      } else if constexpr (OP == OP_INT4) {
        Int4Scale sc = row_sc;
        int lanes_per_group = 64;
        if constexpr (chunk_groups) {
          sc = chunk_sc[c];
        } else if (!row_group) {
          float m = 0.0f;
#pragma unroll
          for (int r = 0; r < S::V; ++r) m = fmaxf(m, fabsf(y[r]));
          lanes_per_group = a.group / S::V;
          sc = int4_scale(group_max(m, lanes_per_group), cnorm, a.scale_dtype);
        }
        const float inv = sc.inv;
        const bool clamp = __builtin_amdgcn_ballot_w64(sc.clamp) != 0;
        uint32_t qb[S::V];
        if (!clamp) {
#pragma unroll
          for (int r = 0; r < S::V; ++r) qb[r] = __float_as_uint(__builtin_fmaf(y[r], inv, 12582912.0f));
        } else {
#pragma unroll
          for (int r = 0; r < S::V; ++r)
            qb[r] = __float_as_uint(__builtin_amdgcn_fmed3f(y[r] * inv, -8.0f, 7.0f) + 12582912.0f);
        }
        if (live) {
          if constexpr (S::V == 16) {
            st_stream(a.packed + (g0 >> 1), pack8_nibbles(qb), pack8_nibbles(qb + 8));
          } else {
            st_stream(a.packed + (g0 >> 1), pack8_nibbles(qb));
          }
          const bool writer = row_group      ? (c == 0 && lane == 0)
                              : chunk_groups ? (lane == 0 && c % (a.group / S::CHUNK) == 0)
                                             : ((lane & (lanes_per_group - 1)) == 0);
          if (writer) {
            const int64_t gi = row_group ? u : (g0 >> __builtin_ctz((unsigned)a.group));
            if (a.scale_dtype == RHTQ_SCALE_F32) static_cast<float*>(a.scales)[gi] = sc.s;
            else static_cast<__half*>(a.scales)[gi] = __float2half_rn(fminf(sc.s, 65504.0f));
          }
        }
      } else if constexpr (OP == OP_NVFP4) {
        // 16-element blocks: one lane (V = 16) or two lanes (V = 8)
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < S::V; ++r) m = fmaxf(m, fabsf(y[r]));
        m = group_max(m, 16 / S::V);
        const uint32_t code = e4m3_code((m * cnorm) * inv6g);
        const float seff = e4m3_value(code) * gts;
        const float inv = seff > 0.0f ? cnorm * __builtin_amdgcn_rcpf(seff) : 0.0f;
        uint32_t words[S::V / 8];
#pragma unroll
        for (int w = 0; w < S::V / 8; ++w) {
          uint32_t acc = 0;
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * w + 0] * inv, y[8 * w + 1] * inv, 1.0f, 0);
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * w + 2] * inv, y[8 * w + 3] * inv, 1.0f, 1);
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * w + 4] * inv, y[8 * w + 5] * inv, 1.0f, 2);
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * w + 6] * inv, y[8 * w + 7] * inv, 1.0f, 3);
          words[w] = seff > 0.0f ? acc : 0u;     // a block whose scale decodes to 0 stores code 0
        }
        if (live) {
          if constexpr (S::V == 16)
            st_stream(a.packed + (g0 >> 1), words[0], words[1]);
          else
            st_stream(a.packed + (g0 >> 1), words[0]);
          if (S::V == 16 || (lane & 1) == 0) static_cast<uint8_t*>(a.scales)[g0 >> 4] = (uint8_t)code;
        }
      } else if constexpr (OP == OP_MXFP4) {
        // 32-element blocks over two lanes (V = 16) or four lanes (V = 8); E8M0 exponent
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < S::V; ++r) m = fmaxf(m, fabsf(y[r]));
        m = group_max(m, 32 / S::V);
        const int ex = mx_exponent(m * cnorm);
        const float inv = m > 0.0f ? __builtin_ldexpf(cnorm, -ex) : 0.0f;
        uint32_t words[S::V / 8];
#pragma unroll
        for (int w = 0; w < S::V / 8; ++w) {
          uint32_t acc = 0;
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * w + 0] * inv, y[8 * w + 1] * inv, 1.0f, 0);
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * w + 2] * inv, y[8 * w + 3] * inv, 1.0f, 1);
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * w + 4] * inv, y[8 * w + 5] * inv, 1.0f, 2);
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, y[8 * w + 6] * inv, y[8 * w + 7] * inv, 1.0f, 3);
          words[w] = inv > 0.0f ? acc : 0u;     // an all-zero block stores code 0
        }
        if (live) {
          if constexpr (S::V == 16)
            st_stream(a.packed + (g0 >> 1), words[0], words[1]);
          else
            st_stream(a.packed + (g0 >> 1), words[0]);
          if ((lane & (32 / S::V - 1)) == 0) static_cast<uint8_t*>(a.scales)[g0 >> 5] = (uint8_t)(ex + 127);
        }
      }
    }
  }

  if constexpr (OP == OP_AMAX) {
    run_max = group_max(run_max, 64);
    __shared__ float wmax[kWaves];
    if (lane == 0) wmax[wave] = run_max;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = wmax[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m = fmaxf(m, wmax[w]);
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale), __float_as_uint(nvfp4_tensor_scale(m * cnorm)));
    }
  }
}

template <int F, int LOGM, int OP, bool CG, int IN>
hipError_t launch_kern(const KernelArgs& a, hipStream_t s);

template <int F, int LOGM, int OP, int IN>
hipError_t launch_one(const KernelArgs& a, hipStream_t s) {
  using S = Shape<F, LOGM>;
  if constexpr (OP == OP_INT4) {
    // per-token, groups inside a chunk, or groups of whole chunks (the API admits powers of two
    // that divide the row)
    if (!(a.group == S::N || a.group <= S::CHUNK || (S::RPU == 1 && a.group < S::N))) return hipErrorNotSupported;
  }
  if constexpr (OP == OP_INT4 && S::RPU == 1 && S::N > S::CHUNK) {
    if (a.group > S::CHUNK && a.group < S::N) return launch_kern<F, LOGM, OP, true, IN>(a, s);
  }
  return launch_kern<F, LOGM, OP, false, IN>(a, s);
}

template <int F, int LOGM, int OP, bool CG, int IN>
hipError_t launch_kern(const KernelArgs& a, hipStream_t s) {
  using S = Shape<F, LOGM>;
  auto kern = fast_kernel<F, LOGM, OP, CG, IN == RHTQ_IN_F32, IN == RHTQ_IN_F16>;
  const int slices = sign_slices<S>(a.sign_period);
  const size_t lds = (size_t)slices * S::NF * 64 * 16 + (size_t)kWaves * S::TBUF * 4;
  if (lds > 65536) return hipErrorNotSupported;
  static const int max_blocks = resident_blocks((const void*)kern, kThreads, lds);
  const int64_t units = (a.rows + S::RPU - 1) / S::RPU;
  const int64_t want = (units + kWaves - 1) / kWaves;
  const int grid = (int)(want < max_blocks ? want : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int OP, int IN>
hipError_t dispatch(const KernelArgs& a, hipStream_t s) {
  switch (a.n) {
    case 16: return launch_one<1, 4, OP, IN>(a, s);
    case 32: return launch_one<1, 5, OP, IN>(a, s);
    case 64: return launch_one<1, 6, OP, IN>(a, s);
    case 128: return launch_one<1, 7, OP, IN>(a, s);
    case 256: return launch_one<1, 8, OP, IN>(a, s);
    case 512: return launch_one<1, 9, OP, IN>(a, s);
    case 1024: return launch_one<1, 10, OP, IN>(a, s);
    case 2048: return launch_one<1, 11, OP, IN>(a, s);
    case 4096: return launch_one<1, 12, OP, IN>(a, s);
    case 8192: return launch_one<1, 13, OP, IN>(a, s);
    case 3072: return launch_one<12, 8, OP, IN>(a, s);
    case 6144: return launch_one<12, 9, OP, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}

template <int IN>
hipError_t dispatch_op(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return dispatch<OP_ROTATE, IN>(a, s);
    case OP_INT4: return dispatch<OP_INT4, IN>(a, s);
    case OP_NVFP4: return dispatch<OP_NVFP4, IN>(a, s);
    case OP_MXFP4: return dispatch<OP_MXFP4, IN>(a, s);
    case OP_AMAX: return dispatch<OP_AMAX, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_fast_f32(int op, const KernelArgs& a, hipStream_t s) {
  if (getenv_fast_disabled()) return hipErrorNotSupported;
  if (a.n == 12288) return launch_fast12_f32(op, a, s);
  if (a.n == 22016 || a.n == 11008 || a.n == 5504 || a.n == 2752) return launch_fast172_f32(op, a, s);
  if (a.n == 16384) return launch_fastw_f32(op, a, s);
  if (a.n == 24576) return launch_fast24_f32(op, a, s);
  return dispatch_op<RHTQ_IN_F32>(op, a, s);
}

hipError_t launch_fast(int op, const KernelArgs& a, hipStream_t s, bool f16in) {
  if (getenv_fast_disabled()) return hipErrorNotSupported;
  if (a.n == 12288) return launch_fast12(op, a, s, f16in);
  if (a.n == 24576) return launch_fast24(op, a, s, f16in);
  if (a.n == 22016 || a.n == 11008 || a.n == 5504 || a.n == 2752) return launch_fast172(op, a, s, f16in);
  if (a.n == 8192 || a.n == 16384) {
    const hipError_t e = launch_fastw(op, a, s, f16in);
    if (e != hipErrorNotSupported) return e;
  }
  if (!getenv_fast2_disabled()) {
    const hipError_t e = launch_fast2(op, a, s, f16in);
    if (e != hipErrorNotSupported) return e;
  }
  return f16in ? dispatch_op<RHTQ_IN_F16>(op, a, s) : dispatch_op<RHTQ_IN_BF16>(op, a, s);
}

}  // namespace rhtq
