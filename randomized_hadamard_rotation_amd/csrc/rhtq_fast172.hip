// Matrix-core kernel for bf16 rows of 11008 = 172 x 64 elements, the Llama 2 7B intermediate
// width (QuaRot reviews, review 2 Questions: its non-power-of-two part 172 makes the rotation
// costly), and of 5504 = 172 x 32 and 2752 = 172 x 16 taken two and four rows at a time (see
// rows172).  Element
// j = 64 a + b (a < 172, b < 64) and
//
//     Y[a'][b''] = sum_a sum_b H172[a'][a] H64[b''][b] s[a][b] x[a][b] / sqrt(11008).
//
// The order-172 factor has no fast algorithm, so it is a dense contraction and runs on the
// matrix cores.  One workgroup of four waves owns one row at a time (persistent grid):
//
//  1. The row (172 x 128 bytes) arrives by 16-byte loads issued one row ahead; the random
//     signs are XORed onto the bf16 sign bits (masks in LDS) and the row is written to LDS
//     transposed, as 64 rows b of 192 bf16 (a contiguous, a >= 172 zero); row b starts at
//     528 b + 16 ((b >> 3) & 7) bytes.  The pitch (4 mod 32 dwords) puts the rows of one
//     16-byte read on distinct banks, and the shift does the same for the eight rows b = 8 k + e
//     of one 2-byte write, so neither conflicts.
//  2. Stage 1, H172 over a, exact on the bf16 input: v_mfma_f32_16x16x32_bf16 with
//     A = X^T (M = b, K = a), one 16-byte LDS read per fragment, and B = H172^T
//     (K = a, N = a'), a +-1 operand held in registers.  K slot e of lane group g stands for
//     a = 32 ks + 8 g + e.  Wave w owns the output tiles a' in [16 t, 16 t + 16),
//     t = w, w + 4, w + 8 (11 tiles, 172 padded to 176).  Result D1[b][a']: lane l holds
//     a' = 16 t + (l & 15) (t the tile) and b = 16 mt + 4 (l >> 4) + i in tile mt, register i.
//  3. Stage 2, H64 = H2 (x) H32 over b: index bit 5 (mt >> 1) is a register butterfly, the
//     other five bits one v_mfma_f32_16x16x32_f16 with A = H32 (M = b''_lo, K = b_lo) and
//     B = the butterflied values, whose registers already are that B layout (slot e of lane
//     group g is b_lo = 16 (e >> 2) + 4 g + (e & 3)).  fp32 does not fit an f16 operand, so
//     each value u is split as u S = hi + lo (two f16 terms, S a power of two per output
//     column a' with |u S| < 2^15) and both halves accumulate through the same operand:
//     22 significant bits.
//  4. Output D2[b''][a']: lane l holds a' = 16 t + (l & 15) and, in run r = 2 hb + mt2,
//     b'' = 16 r + 4 (l >> 4) + i.  Groups of 16 and 32 are runs, groups of 64..256 are
//     1..4 consecutive a' (lane bits 0-1); maxima by lane swaps and DPP.  INT4 codes by the
//     magic-constant FMA, E2M1 by v_cvt_scalef32_pk_fp4_f32; two lane swaps (lane groups
//     g ^ 1, then g ^ 2) leave lane group g with run g whole, so each store instruction writes
//     sixteen complete 32-byte a'-rows.
#include <hip/hip_fp16.h>

#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

// Waves per workgroup.  Four (tiles 3, 3, 3, 2) beat eleven (one tile each, 94-100 VGPRs): every
// wave reads the row's A fragments from LDS for its own tiles, so eleven waves read 2.75 times
// the LDS bytes per row, and LDS bandwidth, not latency, then limits the kernel.
#ifndef RHTQ_172_WAVES
#define RHTQ_172_WAVES 4
#endif
constexpr int kTiles = 11;                       // 16-wide a'-tiles: 172 padded to 176
constexpr int kW = RHTQ_172_WAVES;               // waves per workgroup: wave w owns tiles w, w + kW, ..
constexpr int kT = 64 * kW;
constexpr int kNT = (kTiles + kW - 1) / kW;      // tiles of the busiest wave
constexpr int kN = 11008;                        // 172 x 64
constexpr int kPitch = 528;                      // LDS bytes per b-row: 192 bf16, shift, pad
constexpr int kXBytes = 64 * kPitch;
__host__ __device__ constexpr int xrow(int b) { return b * kPitch + 16 * ((b >> 3) & 7); }
constexpr int kChunks = kN / 8;                  // 16-byte chunks per row
constexpr int kLoads = (kChunks + kT - 1) / kT;  // loads per thread and row

// Stage-1 B operand for output tile t and K-step ks, as a compile-time table (one 16-byte load
// per operand; built lane by lane from bits, each entry cost a dependent load at kernel start):
// slot e of lane group g stands for a = 32 ks + 8 g + e, column n = lane & 15 for
// a' = 16 t + n; H172[a'][a] as bf16 +-1, zero outside 172 x 172.
struct H172TOperands {
  uint16_t v[kTiles][6][64][8];
  constexpr H172TOperands() : v() {
    for (int t = 0; t < kTiles; ++t)
      for (int ks = 0; ks < 6; ++ks)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e) {
            const int ap = 16 * t + (lane & 15), k = 32 * ks + 8 * (lane >> 4) + e;
            v[t][ks][lane][e] = (k < 172 && ap < 172) ? (h172_entry(ap, k) < 0 ? 0xBF80 : 0x3F80) : 0;
          }
  }
};
// The same operands as f16 (+-1 and 0 are exact in both) for fp16 input.
struct H172TOperandsF16 {
  uint16_t v[kTiles][6][64][8];
  constexpr H172TOperandsF16() : v() {
    const H172TOperands h;
    for (int t = 0; t < kTiles; ++t)
      for (int ks = 0; ks < 6; ++ks)
        for (int lane = 0; lane < 64; ++lane)
          for (int e = 0; e < 8; ++e) {
            const uint16_t b = h.v[t][ks][lane][e];
            v[t][ks][lane][e] = b ? (uint16_t)((b & 0x8000) | 0x3C00) : (uint16_t)0;
          }
  }
};
__constant__ H172TOperands kH172TOps;
__constant__ H172TOperandsF16 kH172TOpsF16;

template <bool H16>
__device__ __forceinline__ bf16x8 h172t_operand(int lane, int t, int ks) {
  bf16x8 r;
  if constexpr (H16) __builtin_memcpy(&r, &kH172TOpsF16.v[t][ks][lane][0], 16);
  else __builtin_memcpy(&r, &kH172TOps.v[t][ks][lane][0], 16);
  return r;
}

// Stage-2 A operand for M-tile mt2: row m = lane & 15 stands for b''_lo = 16 mt2 + m, slot e
// of lane group g for b_lo = 16 (e >> 2) + 4 g + (e & 3); entry H32[b''_lo][b_lo] as f16, or with
// I2 == true the block-diagonal I2 (x) H16 (zero where bit 4 of b''_lo and b_lo differ).
template <bool I2 = false>
__device__ f16x8 h32_b_operand(int lane, int mt2) {
  const int m = 16 * mt2 + (lane & 15), g = lane >> 4;
  uint16_t bits[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = 16 * (e >> 2) + 4 * g + (e & 3);
    bits[e] = (I2 && ((m ^ k) & 16)) ? 0 : ((__builtin_popcount(m & k & (I2 ? 15 : 31)) & 1) ? 0xBC00 : 0x3C00);
  }
  f16x8 r;
  __builtin_memcpy(&r, bits, 16);
  return r;
}

// Maximum over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) of non-negative values.
__device__ __forceinline__ float col_max(float v) {
  uint32_t u = __float_as_uint(v);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = umax(p[0], p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(umax(q[0], q[1]));
}

// Maximum of two non-negative floats as unsigned bit patterns (no canonicalisation needed).
__device__ __forceinline__ float nnmax(float a, float b) { return __uint_as_float(umax(__float_as_uint(a), __float_as_uint(b))); }

// P: rows of 11008 / P = 172 x (64 / P) elements per 11008-element work row (1, 2 or 4).  With
// P > 1, P consecutive rows share a work row: b = (64 / P) r + b' holds element (64 / P) a + b'
// of row r of the set.  Stage 1 is per column b and unchanged.  Stage 2 drops the bit-5 butterfly
// (H1 (x) H32 for P = 2) and, for P = 4, also splits the matrix-core product into I2 (x) H16; every
// row gets its own split scale.  The epilogue maps output run r (16 b'' values) to row
// r / (4 / P) of the set.
// GC: group class, 0 (one INT4 group per row: the row maximum across the four waves through
// LDS), 4 (16-element groups: one run), 5 (32: two runs), 6 (64..256: whole
// a'-rows); SD: INT4 scale storage (RHTQ_SCALE_F32 / F16).  H16: fp16 input (stage 1 on the f16
// matrix-core instruction against f16 operands; everything else is the same).  F32: fp32 input,
// taken through the LDS tile in three passes (f32_term: the exact bf16 terms hi, mid, lo of each
// value) that stage 1 accumulates into the same products; the next row's loads are issued
// before the last pass instead of a row ahead (P = 1), or each pass loads its data (P > 1).
template <int P, int OP, int GC, int SD, int NT, bool H16, bool F32>
__device__ __forceinline__ void rows172(const KernelArgs& a, uint8_t* xs, const uint4* sgn, float* wmax) {
  static_assert(P == 1 || P == 2 || P == 4, "one, two or four rows per work row");
  constexpr int kPn = kN / P;     // elements per row
  constexpr int kM = 64 / P;      // b' per row (elements per a'-row)
  constexpr int RPP = 4 / P;      // output runs of 16 per row
  constexpr int LM = P == 1 ? 6 : (P == 2 ? 5 : 4);   // log2 kM
  // split scale of run r: one per work row (P = 1), per half (P = 2) or per run (P = 4)
  auto sidx = [](int r) { return P == 1 ? 0 : (P == 2 ? (r >> 1) : r); };
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, n = lane & 15;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)kPn));
  const int64_t vrows = (a.rows + P - 1) / P;   // work rows
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const float* xf = static_cast<const float*>(a.x);

  bf16x8 hb[NT][6];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) hb[j][ks] = h172t_operand<H16>(lane, wave + kW * j, ks);
  const f16x8 ha[2] = {h32_b_operand<P == 4>(lane, 0), h32_b_operand<P == 4>(lane, 1)};

  float gts = 0.0f, inv6g = 0.0f;
  if constexpr (OP == OP_NVFP4) {
    gts = a.tensor_scale[0];
    inv6g = gts > 0.0f ? 1.0f / (6.0f * gts) : 0.0f;
  }
  const int LG = GC == 6 ? __builtin_ctz((unsigned)a.group) : GC;   // log2 of the group
  float run_max = 0.0f;

  uint4 raw[F32 ? 1 : kLoads];
  uint4 raw32[F32 ? kLoads : 1][2];   // fp32 input: the chunk's 8 values as two 16-byte loads
  auto load = [&](int64_t row) {
    if (row >= vrows) return;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int c = tid + kT * k;
      if (c < kChunks) {
        if constexpr (F32) {
          // as below, with two 16-byte loads of fp32 values per chunk
          const int b0 = 8 * (c & 7);
          const int64_t prow = P == 1 ? row : row * P + b0 / kM;
          const int64_t off = P == 1 ? row * kN + 8 * c : prow * kPn + kM * (c >> 3) + b0 % kM;
          raw32[k][0] = raw32[k][1] = make_uint4(0, 0, 0, 0);
          if (P == 1 || prow < a.rows) {
            raw32[k][0] = ld_stream(xf + off);
            raw32[k][1] = ld_stream(xf + off + 4);
          }
        } else if constexpr (P == 1) {
          raw[k] = ld_stream(x + row * kN + 8 * c);
        } else {
          // chunk c: a = c >> 3, b = 8 (c & 7) .. + 7 of the work row, i.e. row P row + b / kM
          // of the call, elements kM a + b % kM; a row past the end reads as zeros
          const int b0 = 8 * (c & 7);
          const int64_t prow = row * P + b0 / kM;
          raw[k] = prow < a.rows ? ld_stream(x + prow * kPn + kM * (c >> 3) + b0 % kM) : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  int64_t row = blockIdx.x;
  load(row);

  // this thread's chunks c = tid + kT k hold a = (tid >> 3) + (kT / 8) k and b = 8 (tid & 7) + e
  uint8_t* wbase = xs + xrow(8 * (tid & 7)) + 2 * (tid >> 3);
  // fragment (ks, mt) of this lane: row b = 16 mt + n, a = 32 ks + 8 g .. + 7
  const uint8_t* rbase_l[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) rbase_l[mt] = xs + xrow(16 * mt + n) + 16 * g;
  // x of the row in raw[] -> LDS, signs applied; fp32 input: bf16 term `term` of each value
  auto write_lds = [&](int term) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int c = tid + kT * k;
      if (c < kChunks) {
        const uint4 m = sgn[c];
        if constexpr (F32) {
          const uint32_t mk[4] = {m.x, m.y, m.z, m.w};
          const uint4 r0 = raw32[k][0], r1 = raw32[k][1];
          const uint32_t v[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // the sign flips the whole fp32 value (bit 15 / bit 31 of the bf16-pair mask)
            const uint32_t sb = (e & 1) ? (mk[e >> 1] & 0x80000000u) : (mk[e >> 1] << 16);
            *reinterpret_cast<uint16_t*>(wbase + e * kPitch + (kT / 4) * k) = (uint16_t)(f32_term(v[e] ^ sb, term) >> 16);
          }
        } else {
          const uint32_t w[4] = {raw[k].x ^ m.x, raw[k].y ^ m.y, raw[k].z ^ m.z, raw[k].w ^ m.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint16_t*>(wbase + e * kPitch + (kT / 4) * k) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  };
  // stage 1 (H172 over a) of the tile in LDS, into acc (first: start from zero)
  auto stage1 = [&](f32x4 (&acc)[NT][4], bool first) {
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      bf16x8 av[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) av[mt] = *reinterpret_cast<const bf16x8*>(rbase_l[mt] + 64 * ks);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
          acc[j][mt] = stage1_mma<H16>(av[mt], hb[j][ks], (first && ks == 0) ? z : acc[j][mt]);
        }
    }
  };
  __syncthreads();   // sign masks and zeroed rows
  if (row < vrows) write_lds(0);
  if constexpr (!F32) load(row + gridDim.x);
  __syncthreads();
  // per row: stage 1 reads the row from LDS; after the barrier that ends those reads the next
  // row goes into LDS (its loads were issued one row earlier) and the loads of the row after
  // it are issued, then stage 2 and the epilogue of this row run from registers.  fp32 input:
  // three passes (hi, mid, lo) through the tile, the next row's loads issued before the third
  for (; row < vrows; row += gridDim.x) {
    // ---------------- stage 1: H172 over a ----------------
    f32x4 acc[NT][4];
    stage1(acc, true);
    __syncthreads();   // every wave has read this row
    if constexpr (F32 && P == 1) {
      write_lds(1);
      __syncthreads();
      stage1(acc, false);
      __syncthreads();
      write_lds(2);
      load(row + gridDim.x);
      __syncthreads();
      stage1(acc, false);
      __syncthreads();
      if (row + gridDim.x < vrows) write_lds(0);
    } else if constexpr (F32) {
      // two and four rows per work row leave no registers to hold the fp32 data across a
      // pass: it is loaded again right before each term is written
#pragma unroll 1
      for (int term = 1; term < 3; ++term) {
        load(row);
        write_lds(term);
        __syncthreads();
        stage1(acc, false);
        __syncthreads();
      }
      if (row + gridDim.x < vrows) {
        load(row + gridDim.x);
        write_lds(0);
      }
    } else {
      if (row + gridDim.x < vrows) write_lds(0);
      load(row + 2 * (int64_t)gridDim.x);
    }

    // ---------------- stage 2: H2 by butterfly (P = 1), H32 on the matrix cores ----------------
    // (each step runs over all of this wave's tiles before the next, so that the tiles'
    // independent chains interleave)
    float u[NT][2][2][4];       // [tile][hb][mt & 1][i], b_lo = 16 (mt & 1) + 4 g + i
    float S[NT][4], invS_t[NT][4];   // split scale of run group sidx(r)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (P == 1) {
        float m = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = acc[j][h][i], q = acc[j][h + 2][i];
            u[j][0][h][i] = p + q;
            u[j][1][h][i] = p - q;
            m = fmaxf(m, fmaxf(fabsf(p + q), fabsf(p - q)));
          }
        S[j][0] = m;
      } else if constexpr (P == 2) {
        // half hb is row hb of the pair: no butterfly, a split scale of its own
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          float m = 0.0f;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              u[j][hb][h][i] = acc[j][2 * hb + h][i];
              m = fmaxf(m, fabsf(acc[j][2 * hb + h][i]));
            }
          S[j][hb] = m;
        }
      } else {
        // M-tile 2 hb + h is row 2 hb + h of the set, with a split scale of its own
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              u[j][hb][h][i] = acc[j][2 * hb + h][i];
              m = fmaxf(m, fabsf(acc[j][2 * hb + h][i]));
            }
            S[j][2 * hb + h] = m;
          }
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (P == 1) {
        split_scale(__float_as_uint(col_max(S[j][0])), S[j][0], invS_t[j][0]);
      } else {
#pragma unroll
        for (int q = 0; q < P; ++q) split_scale(__float_as_uint(col_max(S[j][q])), S[j][q], invS_t[j][q]);
      }
    }
    float d2a[NT][4][4];   // [tile][run r = 2 hb + mt2][i]: b'' = 16 r + 4 g + i
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float ys[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ys[e] = u[j][h][e >> 2][e & 3];
        uint32_t hw[4], lw[4];
        if constexpr (P == 4) split8x2(ys, S[j][2 * h], S[j][2 * h + 1], hw, lw);
        else split8(ys, S[j][sidx(2 * h)], hw, lw);
        f16x8 bh, bl;
        __builtin_memcpy(&bh, hw, 16);
        __builtin_memcpy(&bl, lw, 16);
#pragma unroll
        for (int mt2 = 0; mt2 < 2; ++mt2) {
          const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
          f32x4 o = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[mt2], bh, z, 0, 0, 0);
          o = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[mt2], bl, o, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) d2a[j][2 * h + mt2][i] = o[i];
        }
      }

    // per-token INT4: one scale per row, from the maximum over every tile of the four waves
    // (columns a' >= 172 are zero); all waves pass this barrier, GC being uniform
    float row_inv[P] = {};
    bool row_clamp = false;
    if constexpr (OP == OP_INT4 && GC == 0) {
      float m[P] = {};
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float mj = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) mj = fmaxf(mj, fabsf(d2a[j][r][i]));
          m[r / RPP] = nnmax(m[r / RPP], mj * invS_t[j][sidx(r)]);
        }
#pragma unroll
      for (int hh = 0; hh < P; ++hh) {
        m[hh] = group_max(m[hh], 64);
        if (lane == 0) wmax[P * wave + hh] = m[hh];
      }
      __syncthreads();
#pragma unroll
      for (int hh = 0; hh < P; ++hh) {
        float rm = wmax[hh];
#pragma unroll
        for (int w = 1; w < kW; ++w) rm = nnmax(rm, wmax[P * w + hh]);
        const Int4Scale sc = int4_scale(rm, cnorm, SD);
        row_inv[hh] = sc.inv;
        row_clamp |= sc.clamp;
        const int64_t prow = row * P + hh;
        if (tid == 0 && prow < a.rows) {
          if constexpr (SD == RHTQ_SCALE_F32) static_cast<float*>(a.scales)[prow] = sc.s;
          else static_cast<__half*>(a.scales)[prow] = __float2half_rn(fminf(sc.s, 65504.0f));
        }
      }
    }

#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int ap = 16 * (wave + kW * j) + n;
      const bool valid = ap < 172;
      const auto& d2 = d2a[j];
      // run r: row P row + r / RPP of the call, its elements rstart(r) + 4 g + i
      auto prow_of = [&](int r) -> int64_t { return row * P + r / RPP; };
      auto rstart = [&](int r) -> int64_t { return prow_of(r) * kPn + kM * ap + 16 * (r % RPP); };
      auto rvalid = [&](int r) -> bool { return valid && (P == 1 || prow_of(r) < a.rows); };
      if constexpr (OP == OP_ROTATE) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float f = invS_t[j][sidx(r)] * cnorm;
          if (rvalid(r)) st_stream(a.y + rstart(r) + 4 * g, d2[r][0] * f, d2[r][1] * f, d2[r][2] * f, d2[r][3] * f);
        }
        continue;
      }
      float mr[4];   // run maxima, split units
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mr[r] = fmaxf(fmaxf(fabsf(d2[r][0]), fabsf(d2[r][1])), fmaxf(fabsf(d2[r][2]), fabsf(d2[r][3])));
      if constexpr (OP == OP_AMAX) {
#pragma unroll
        for (int r = 0; r < 4; ++r) run_max = nnmax(run_max, mr[r] * invS_t[j][sidx(r)]);
        continue;
      }

      // ---------------- group scales, once per group ----------------
      // sl[r]: factor from split units to code units for run r (0 for an all-zero group)
      float sl[4];
      bool clamp = false;
      // bm: true units, before 1/sqrt(n); invS: the split units of the runs the factor is for
      auto scale_of = [&](float bm, int64_t gi, bool writer, float invS) -> float {
        if constexpr (OP == OP_INT4) {
          const Int4Scale sc = int4_scale(bm, cnorm, SD);
          clamp |= sc.clamp;
          if (writer) {
            if constexpr (SD == RHTQ_SCALE_F32) static_cast<float*>(a.scales)[gi] = sc.s;
            else static_cast<__half*>(a.scales)[gi] = __float2half_rn(fminf(sc.s, 65504.0f));
          }
          return sc.inv * invS;
        } else if constexpr (OP == OP_NVFP4) {
          const uint32_t code = e4m3_code((bm * cnorm) * inv6g);
          const float seff = e4m3_value(code) * gts;
          if (writer) static_cast<uint8_t*>(a.scales)[gi] = (uint8_t)code;
          return seff > 0.0f ? (cnorm * __builtin_amdgcn_rcpf(seff)) * invS : 0.0f;
        } else {
          const float bt = bm * cnorm;
          const int ex = mx_exponent(bt);
          if (writer) static_cast<uint8_t*>(a.scales)[gi] = (uint8_t)(ex + 127);
          return bt > 0.0f ? __builtin_ldexpf(invS * cnorm, -ex) : 0.0f;
        }
      };
      if constexpr (GC == 0) {   // the row's scale, in the runs' split units
#pragma unroll
        for (int r = 0; r < 4; ++r) sl[r] = row_inv[r / RPP] * invS_t[j][sidx(r)];
        clamp = row_clamp;
      } else if constexpr (GC == 4) {   // a run per group; lane group g stores the scale of run g
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sl[r] = scale_of(col_max(mr[r]) * invS_t[j][sidx(r)], rstart(r) >> 4, rvalid(r) && g == r, invS_t[j][sidx(r)]);
      } else if constexpr (P == 4) {   // 2 or 4 whole 16-element a'-rows of one row; lane group r stores for run r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float mm = col_max(mr[r]) * invS_t[j][r];
          mm = dpp_max<0xB1>(mm);                 // a' pairs (lane xor 1)
          if (LG >= 6) mm = dpp_max<0x4E>(mm);    // a' quads (lane xor 2)
          sl[r] = scale_of(mm, rstart(r) >> LG, rvalid(r) && g == r && (ap & ((1 << (LG - LM)) - 1)) == 0,
                           invS_t[j][r]);
        }
      } else if constexpr (GC == 5) {   // two runs per group; lane groups 0 and 1 store
        const float s0 = scale_of(col_max(nnmax(mr[0], mr[1])) * invS_t[j][sidx(0)], rstart(0) >> 5,
                                  rvalid(0) && g == 0, invS_t[j][sidx(0)]);
        const float s1 = scale_of(col_max(nnmax(mr[2], mr[3])) * invS_t[j][sidx(2)], rstart(2) >> 5,
                                  rvalid(2) && g == 1, invS_t[j][sidx(2)]);
        sl[0] = sl[1] = s0;
        sl[2] = sl[3] = s1;
      } else if constexpr (P == 1) {   // 1, 2 or 4 whole a'-rows per group; lane group 0 of the group's first a' stores
        float mm = col_max(nnmax(nnmax(mr[0], mr[1]), nnmax(mr[2], mr[3]))) * invS_t[j][0];
        if (LG >= 7) mm = dpp_max<0xB1>(mm);   // a' pairs (lane xor 1)
        if (LG >= 8) mm = dpp_max<0x4E>(mm);   // a' quads (lane xor 2)
        const float s0 = scale_of(mm, rstart(0) >> LG, valid && g == 0 && (ap & ((1 << (LG - 6)) - 1)) == 0,
                                  invS_t[j][0]);
        sl[0] = sl[1] = sl[2] = sl[3] = s0;
      } else {   // P = 2: 2 or 4 whole 32-element a'-rows of one row per group
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float mm = col_max(nnmax(mr[2 * hh], mr[2 * hh + 1])) * invS_t[j][sidx(2 * hh)];
          mm = dpp_max<0xB1>(mm);                 // a' pairs (lane xor 1)
          if (LG >= 7) mm = dpp_max<0x4E>(mm);    // a' quads (lane xor 2)
          const float sh = scale_of(mm, rstart(2 * hh) >> LG,
                                    rvalid(2 * hh) && g == 0 && (ap & ((1 << (LG - LM)) - 1)) == 0,
                                    invS_t[j][sidx(2 * hh)]);
          sl[2 * hh] = sl[2 * hh + 1] = sh;
        }
      }

      // ---------------- codes: runs 0,1 -> p01, runs 2,3 -> p23 (run in 16-bit halves) ----------------
      uint32_t p01, p23;
      if constexpr (OP == OP_INT4) {
        const bool any_clamp = __builtin_amdgcn_ballot_w64(clamp) != 0;
        uint32_t q[4][4];
        if (!any_clamp) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) q[r][i] = __float_as_uint(__builtin_fmaf(d2[r][i], sl[r], 12582912.0f));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              q[r][i] = __float_as_uint(__builtin_amdgcn_fmed3f(d2[r][i] * sl[r], -8.0f, 7.0f) + 12582912.0f);
        }
        const uint32_t q01[8] = {q[0][0], q[0][1], q[0][2], q[0][3], q[1][0], q[1][1], q[1][2], q[1][3]};
        const uint32_t q23[8] = {q[2][0], q[2][1], q[2][2], q[2][3], q[3][0], q[3][1], q[3][2], q[3][3]};
        p01 = pack8_nibbles(q01);
        p23 = pack8_nibbles(q23);
      } else {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            const int r = 2 * h + rr;
            const float s = sl[r];
            uint32_t t = 0;
            t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, d2[r][0] * s, d2[r][1] * s, 1.0f, 0);
            t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, d2[r][2] * s, d2[r][3] * s, 1.0f, 1);
            w[h] |= (s > 0.0f ? (t & 0xFFFFu) : 0u) << (16 * rr);   // zero-scale group -> code 0
          }
        }
        p01 = w[0];
        p23 = w[1];
      }
      // lane group g keeps runs g & 1 and 2 + (g & 1), sends the other two to g ^ 1 and
      // receives the partner's halves of its own runs: eight consecutive codes per dword
      const bool odd = g & 1;
      const uint32_t send = __builtin_amdgcn_perm(p23, p01, odd ? 0x05040100u : 0x07060302u);
      const uint32_t keep = __builtin_amdgcn_perm(p23, p01, odd ? 0x07060302u : 0x05040100u);
      auto pr = __builtin_amdgcn_permlane16_swap(send, send, false, false);
      const uint32_t recv = odd ? pr[0] : pr[1];
      const uint32_t lo = odd ? recv : keep, hi = odd ? keep : recv;
      // now w0 holds bytes 2 (g & 2) + 8 (g & 1) .. + 3 of the a'-row and w1 the same + 16; lane
      // groups g and g ^ 2 trade once more so that lane group g holds bytes 8 g .. 8 g + 7
      const uint32_t w0 = __builtin_amdgcn_perm(hi, lo, 0x05040100u), w1 = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
      const bool upper = g & 2;
      const uint32_t send2 = upper ? w0 : w1;
      auto pr2 = __builtin_amdgcn_permlane32_swap(send2, send2, false, false);
      const uint32_t recv2 = upper ? pr2[0] : pr2[1];
      // lane group g: bytes 8 g .. 8 g + 7 of the work row's 32-byte a'-row, i.e. of row P row + g / (4 / P)
      const int rg = g / (4 / P);
      if (rvalid(RPP * rg))
        st_stream(a.packed + ((prow_of(RPP * rg) * kPn + kM * ap) >> 1) + 8 * (g % (4 / P)), upper ? recv2 : w0,
                  upper ? w1 : recv2);
    }
    __syncthreads();   // the next row is in LDS
  }

  if constexpr (OP == OP_AMAX) {
    run_max = group_max(run_max, 64);
    if (lane == 0) wmax[wave] = run_max;
    __syncthreads();
    if (tid == 0) {
      float mm = wmax[0];
#pragma unroll
      for (int w = 1; w < kW; ++w) mm = nnmax(mm, wmax[w]);
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale), __float_as_uint(nvfp4_tensor_scale(mm * cnorm)));
    }
  }
}

template <int P, int OP, int GC, int SD, bool H16 = false, bool F32 = false>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(kW == 4 ? 2 : 4))) void fast172_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kXBytes];
  __shared__ uint4 sgn[kChunks];
  __shared__ float wmax[kW * P];
  const int tid = threadIdx.x;
  for (int c = tid; c < kChunks; c += kT) {
    uint4 m = make_uint4(0, 0, 0, 0);
    if (a.signs) {
      // chunk c of the work row: elements kM a + b % kM of one row of the pair (rows share the signs)
      constexpr int kM = 64 / P;
      const int b0 = 8 * (c & 7);
      const uint2 sv = *reinterpret_cast<const uint2*>(a.signs + kM * (c >> 3) + b0 % kM);
      m.x = __builtin_amdgcn_perm(0u, sv.x, 0x010C000Cu) & 0x80008000u;
      m.y = __builtin_amdgcn_perm(0u, sv.x, 0x030C020Cu) & 0x80008000u;
      m.z = __builtin_amdgcn_perm(0u, sv.y, 0x010C000Cu) & 0x80008000u;
      m.w = __builtin_amdgcn_perm(0u, sv.y, 0x030C020Cu) & 0x80008000u;
    }
    sgn[c] = m;
  }
  for (int c = tid; c < kXBytes / 16; c += kT) reinterpret_cast<uint4*>(xs)[c] = make_uint4(0, 0, 0, 0);   // a >= 172 stays 0
  // waves with a tile fewer than the busiest (kTiles not a multiple of kW) take the smaller copy
  if constexpr (kTiles % kW == 0) {
    rows172<P, OP, GC, SD, kNT, H16, F32>(a, xs, sgn, wmax);
  } else {
    if ((tid >> 6) < kTiles % kW) rows172<P, OP, GC, SD, kNT, H16, F32>(a, xs, sgn, wmax);
    else rows172<P, OP, GC, SD, kNT - 1, H16, F32>(a, xs, sgn, wmax);
  }
}

// ---------------------------------------------------------------------------
// 22016 = 172 x 128 (H172 (x) H128): element j = 128 a + b, b < 128.  H128 = H2 (x) H64 with
// the top bit c of b = 64 c + d outer, and the factors commute, so a row is its two halves
// c = 0, 1 (172 x 64 each, element 128 a + 64 c + d), each taken through the same LDS buffer
// and the same stage 1 (H172 over a) as an 11008 row; one butterfly between the two halves'
// stage-1 results applies the H2, and each half then runs the 11008 stage 2 (H64 over d) and
// epilogue on its own output half-row 128 a' + 64 c' + [0, 64).  Groups of 64 lie in a half,
// groups of 128 .. 512 are 1 .. 4 whole a'-rows (both halves); the per-token maximum spans both.
// ---------------------------------------------------------------------------
constexpr int kN2 = 2 * kN;          // 22016
constexpr int kChunks2 = 2 * kChunks;

// F32: fp32 input; each half goes through the LDS tile in three passes (the bf16 terms of
// f32_term, accumulated into the same products), and each pass loads its half again right
// before writing it, so no fp32 data is held across a pass.
template <int OP, int GC, int SD, int NT, bool H16, bool F32>
__device__ __forceinline__ void rows344(const KernelArgs& a, uint8_t* xs, const uint4* sgn, float* wmax) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, n = lane & 15;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)kN2));
  const int64_t rows = a.rows;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const float* xf = static_cast<const float*>(a.x);

  const f16x8 ha[2] = {h32_b_operand<false>(lane, 0), h32_b_operand<false>(lane, 1)};

  float gts = 0.0f, inv6g = 0.0f;
  if constexpr (OP == OP_NVFP4) {
    gts = a.tensor_scale[0];
    inv6g = gts > 0.0f ? 1.0f / (6.0f * gts) : 0.0f;
  }
  const int LG = GC == 6 ? __builtin_ctz((unsigned)a.group) : GC;   // log2 of the group
  float run_max = 0.0f;

  // half h of a row: chunk c < kChunks holds a = c >> 3 and d = 8 (c & 7) .. + 7, the elements
  // 128 a + 64 h + d
  uint4 raw[F32 ? 1 : kLoads];
  uint4 raw32[F32 ? kLoads : 1][2];
  auto load = [&](int64_t row, int h) {
    if (row >= rows) return;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int c = tid + kT * k;
      if constexpr (F32) {
        if (c < kChunks) {
          const float* p = xf + row * kN2 + 128 * (c >> 3) + 64 * h + 8 * (c & 7);
          raw32[k][0] = ld_stream(p);
          raw32[k][1] = ld_stream(p + 4);
        }
      } else {
        if (c < kChunks) raw[k] = ld_stream(x + row * kN2 + 128 * (c >> 3) + 64 * h + 8 * (c & 7));
      }
    }
  };
  uint8_t* wbase = xs + xrow(8 * (tid & 7)) + 2 * (tid >> 3);
  const uint8_t* rbase_l[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) rbase_l[mt] = xs + xrow(16 * mt + n) + 16 * g;
  auto write_lds = [&](int h, int term) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int c = tid + kT * k;
      if (c < kChunks) {
        const uint4 m = sgn[kChunks * h + c];
        if constexpr (F32) {
          const uint32_t mk[4] = {m.x, m.y, m.z, m.w};
          const uint4 r0 = raw32[k][0], r1 = raw32[k][1];
          const uint32_t v[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t sb = (e & 1) ? (mk[e >> 1] & 0x80000000u) : (mk[e >> 1] << 16);
            *reinterpret_cast<uint16_t*>(wbase + e * kPitch + (kT / 4) * k) = (uint16_t)(f32_term(v[e] ^ sb, term) >> 16);
          }
        } else {
          const uint32_t w[4] = {raw[k].x ^ m.x, raw[k].y ^ m.y, raw[k].z ^ m.z, raw[k].w ^ m.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint16_t*>(wbase + e * kPitch + (kT / 4) * k) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  };
  // stage 1 (H172 over a) of the half in LDS; the H172^T operands are loaded (L2 hits) for each
  // pass rather than held, which leaves the registers to the two halves' results
  auto stage1 = [&](f32x4 (&acc)[NT][4], bool first) {
    // an opaque zero keeps the compiler from hoisting these loads out of the row loop
    int t0 = wave;
    asm volatile("" : "+v"(t0));
    bf16x8 hb[NT][6];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) hb[j][ks] = h172t_operand<H16>(lane, t0 + kW * j, ks);
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      bf16x8 av[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) av[mt] = *reinterpret_cast<const bf16x8*>(rbase_l[mt] + 64 * ks);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
          acc[j][mt] = stage1_mma<H16>(av[mt], hb[j][ks], (first && ks == 0) ? z : acc[j][mt]);
        }
    }
  };
  // fp32 input: half h of the row through the tile, term by term, into acc (the tile is free)
  auto half_f32 = [&](int64_t row, int h, f32x4 (&acc)[NT][4]) {
    load(row, h);
    write_lds(h, 0);
    __syncthreads();
    stage1(acc, true);
    __syncthreads();   // every wave has read the tile
#pragma unroll 1
    for (int term = 1; term < 3; ++term) {
      load(row, h);
      write_lds(h, term);
      __syncthreads();
      stage1(acc, false);
      __syncthreads();
    }
  };

  int64_t row = blockIdx.x;
  if constexpr (!F32) {
    load(row, 0);
    __syncthreads();   // sign masks and zeroed rows
    if (row < rows) write_lds(0, 0);
    load(row, 1);
  }
  __syncthreads();
  // per row: stage 1 of half 0 (in LDS); half 1 (in raw[]) goes in after the barrier that ends
  // those reads, and the next row's half 0 is loaded; stage 1 of half 1; the next row's half 0
  // goes in and its half 1 is loaded; then the H2 butterfly, stage 2 and the epilogue run from
  // registers
  for (; row < rows; row += gridDim.x) {
    f32x4 acc[2][NT][4];
    if constexpr (F32) {
      half_f32(row, 0, acc[0]);
      half_f32(row, 1, acc[1]);
    } else {
      stage1(acc[0], true);
      __syncthreads();   // every wave has read half 0
      write_lds(1, 0);
      load(row + gridDim.x, 0);
      __syncthreads();
      stage1(acc[1], true);
      __syncthreads();   // every wave has read half 1
      if (row + gridDim.x < rows) write_lds(0, 0);
      load(row + gridDim.x, 1);
    }

    // H2 over c: half 0 <- half 0 + half 1, half 1 <- half 0 - half 1
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = acc[0][j][mt][i], q = acc[1][j][mt][i];
          acc[0][j][mt][i] = p + q;
          acc[1][j][mt][i] = p - q;
        }

    // ---------------- stage 2 per half: H2 by butterfly, H32 on the matrix cores ----------------
    float d2a[2][NT][4][4];   // [half][tile][run r][i]: b'' = 16 r + 4 g + i of the half
    float invS_t[2][NT];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float u[NT][2][2][4];
      float S[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = acc[c][j][h][i], q = acc[c][j][h + 2][i];
            u[j][0][h][i] = p + q;
            u[j][1][h][i] = p - q;
            m = fmaxf(m, fmaxf(fabsf(p + q), fabsf(p - q)));
          }
        S[j] = m;
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) split_scale(__float_as_uint(col_max(S[j])), S[j], invS_t[c][j]);
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float ys[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) ys[e] = u[j][h][e >> 2][e & 3];
          uint32_t hw[4], lw[4];
          split8(ys, S[j], hw, lw);
          f16x8 bh, bl;
          __builtin_memcpy(&bh, hw, 16);
          __builtin_memcpy(&bl, lw, 16);
#pragma unroll
          for (int mt2 = 0; mt2 < 2; ++mt2) {
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4 o = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[mt2], bh, z, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha[mt2], bl, o, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) d2a[c][j][2 * h + mt2][i] = o[i];
          }
        }
    }

    // per-token INT4: one scale per row, from the maximum over both halves of every tile of the
    // four waves (columns a' >= 172 are zero); all waves pass this barrier, GC being uniform
    float row_inv = 0.0f;
    bool row_clamp = false;
    if constexpr (OP == OP_INT4 && GC == 0) {
      float m = 0.0f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float mj = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) mj = fmaxf(mj, fabsf(d2a[c][j][r][i]));
            m = nnmax(m, mj * invS_t[c][j]);
          }
      m = group_max(m, 64);
      if (lane == 0) wmax[wave] = m;
      __syncthreads();
      float rm = wmax[0];
#pragma unroll
      for (int w = 1; w < kW; ++w) rm = nnmax(rm, wmax[w]);
      const Int4Scale sc = int4_scale(rm, cnorm, SD);
      row_inv = sc.inv;
      row_clamp = sc.clamp;
      if (tid == 0) {
        if constexpr (SD == RHTQ_SCALE_F32) static_cast<float*>(a.scales)[row] = sc.s;
        else static_cast<__half*>(a.scales)[row] = __float2half_rn(fminf(sc.s, 65504.0f));
      }
    }

#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int ap = 16 * (wave + kW * j) + n;
      const bool valid = ap < 172;
      // run r of half c: elements rstart(c, r) + 4 g + i
      auto rstart = [&](int c, int r) -> int64_t { return row * kN2 + 128 * ap + 64 * c + 16 * r; };
      if constexpr (OP == OP_ROTATE) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float f = invS_t[c][j] * cnorm;
            const float* d = d2a[c][j][r];
            if (valid) st_stream(a.y + rstart(c, r) + 4 * g, d[0] * f, d[1] * f, d[2] * f, d[3] * f);
          }
        continue;
      }
      float mr[2][4];   // run maxima, split units
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float* d = d2a[c][j][r];
          mr[c][r] = fmaxf(fmaxf(fabsf(d[0]), fabsf(d[1])), fmaxf(fabsf(d[2]), fabsf(d[3])));
        }
      if constexpr (OP == OP_AMAX) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) run_max = nnmax(run_max, mr[c][r] * invS_t[c][j]);
        continue;
      }

      // ---------------- group scales, once per group ----------------
      // sl[c][r]: factor from the split units of half c to code units for run r (0 for an
      // all-zero group); scale_of returns that factor for unit split scale (true units)
      float sl[2][4];
      bool clamp = false;
      auto scale_of = [&](float bm, int64_t gi, bool writer) -> float {
        if constexpr (OP == OP_INT4) {
          const Int4Scale sc = int4_scale(bm, cnorm, SD);
          clamp |= sc.clamp;
          if (writer) {
            if constexpr (SD == RHTQ_SCALE_F32) static_cast<float*>(a.scales)[gi] = sc.s;
            else static_cast<__half*>(a.scales)[gi] = __float2half_rn(fminf(sc.s, 65504.0f));
          }
          return sc.inv;
        } else if constexpr (OP == OP_NVFP4) {
          const uint32_t code = e4m3_code((bm * cnorm) * inv6g);
          const float seff = e4m3_value(code) * gts;
          if (writer) static_cast<uint8_t*>(a.scales)[gi] = (uint8_t)code;
          return seff > 0.0f ? cnorm * __builtin_amdgcn_rcpf(seff) : 0.0f;
        } else {
          const float bt = bm * cnorm;
          const int ex = mx_exponent(bt);
          if (writer) static_cast<uint8_t*>(a.scales)[gi] = (uint8_t)(ex + 127);
          return bt > 0.0f ? __builtin_ldexpf(cnorm, -ex) : 0.0f;
        }
      };
      if constexpr (GC == 0) {   // the row's scale, in each half's split units
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) sl[c][r] = row_inv * invS_t[c][j];
        clamp = row_clamp;
      } else if constexpr (GC == 4) {   // a run per group; lane group g stores the scale of run g
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sl[c][r] = scale_of(col_max(mr[c][r]) * invS_t[c][j], rstart(c, r) >> 4, valid && g == r) * invS_t[c][j];
      } else if constexpr (GC == 5) {   // two runs per group; lane groups 0 and 1 store
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const float s0 = scale_of(col_max(nnmax(mr[c][0], mr[c][1])) * invS_t[c][j], rstart(c, 0) >> 5, valid && g == 0);
          const float s1 = scale_of(col_max(nnmax(mr[c][2], mr[c][3])) * invS_t[c][j], rstart(c, 2) >> 5, valid && g == 1);
          sl[c][0] = sl[c][1] = s0 * invS_t[c][j];
          sl[c][2] = sl[c][3] = s1 * invS_t[c][j];
        }
      } else {   // 64: a half a'-row; 128 .. 512: 1 .. 4 whole a'-rows (lane bits 0-1 for a')
        float mh[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
          mh[c] = col_max(nnmax(nnmax(mr[c][0], mr[c][1]), nnmax(mr[c][2], mr[c][3]))) * invS_t[c][j];
        if (LG == 6) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float f = scale_of(mh[c], rstart(c, 0) >> 6, valid && g == 0);
            sl[c][0] = sl[c][1] = sl[c][2] = sl[c][3] = f * invS_t[c][j];
          }
        } else {
          float mm = nnmax(mh[0], mh[1]);
          if (LG >= 8) mm = dpp_max<0xB1>(mm);   // a' pairs (lane xor 1)
          if (LG >= 9) mm = dpp_max<0x4E>(mm);   // a' quads (lane xor 2)
          const float f = scale_of(mm, rstart(0, 0) >> LG, valid && g == 0 && (ap & ((1 << (LG - 7)) - 1)) == 0);
#pragma unroll
          for (int c = 0; c < 2; ++c) sl[c][0] = sl[c][1] = sl[c][2] = sl[c][3] = f * invS_t[c][j];
        }
      }

      // ---------------- codes per half, stored as the half's 32-byte a'-row ----------------
      bool any_clamp = false;
      if constexpr (OP == OP_INT4) any_clamp = __builtin_amdgcn_ballot_w64(clamp) != 0;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const auto& d2 = d2a[c][j];
        uint32_t p01, p23;
        if constexpr (OP == OP_INT4) {
          uint32_t q[4][4];
          if (!any_clamp) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int i = 0; i < 4; ++i) q[r][i] = __float_as_uint(__builtin_fmaf(d2[r][i], sl[c][r], 12582912.0f));
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                q[r][i] = __float_as_uint(__builtin_amdgcn_fmed3f(d2[r][i] * sl[c][r], -8.0f, 7.0f) + 12582912.0f);
          }
          const uint32_t q01[8] = {q[0][0], q[0][1], q[0][2], q[0][3], q[1][0], q[1][1], q[1][2], q[1][3]};
          const uint32_t q23[8] = {q[2][0], q[2][1], q[2][2], q[2][3], q[3][0], q[3][1], q[3][2], q[3][3]};
          p01 = pack8_nibbles(q01);
          p23 = pack8_nibbles(q23);
        } else {
          uint32_t w[2] = {0u, 0u};
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
              const int r = 2 * h + rr;
              const float sv = sl[c][r];
              uint32_t t = 0;
              t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, d2[r][0] * sv, d2[r][1] * sv, 1.0f, 0);
              t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, d2[r][2] * sv, d2[r][3] * sv, 1.0f, 1);
              w[h] |= (sv > 0.0f ? (t & 0xFFFFu) : 0u) << (16 * rr);   // zero-scale group -> code 0
            }
          }
          p01 = w[0];
          p23 = w[1];
        }
        // lane group g keeps runs g & 1 and 2 + (g & 1), sends the other two to g ^ 1 and
        // receives the partner's halves of its own runs, then lane groups g and g ^ 2 trade so
        // that lane group g holds bytes 8 g .. 8 g + 7 of the half's 32-byte a'-row
        const bool odd = g & 1;
        const uint32_t send = __builtin_amdgcn_perm(p23, p01, odd ? 0x05040100u : 0x07060302u);
        const uint32_t keep = __builtin_amdgcn_perm(p23, p01, odd ? 0x07060302u : 0x05040100u);
        auto pr = __builtin_amdgcn_permlane16_swap(send, send, false, false);
        const uint32_t recv = odd ? pr[0] : pr[1];
        const uint32_t lo = odd ? recv : keep, hi = odd ? keep : recv;
        const uint32_t w0 = __builtin_amdgcn_perm(hi, lo, 0x05040100u), w1 = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
        const bool upper = g & 2;
        const uint32_t send2 = upper ? w0 : w1;
        auto pr2 = __builtin_amdgcn_permlane32_swap(send2, send2, false, false);
        const uint32_t recv2 = upper ? pr2[0] : pr2[1];
        if (valid) st_stream(a.packed + ((row * kN2 + 128 * ap + 64 * c) >> 1) + 8 * g, upper ? recv2 : w0, upper ? w1 : recv2);
      }
    }
    __syncthreads();   // the next row's half 0 is in LDS
  }

  if constexpr (OP == OP_AMAX) {
    run_max = group_max(run_max, 64);
    if (lane == 0) wmax[wave] = run_max;
    __syncthreads();
    if (tid == 0) {
      float mm = wmax[0];
#pragma unroll
      for (int w = 1; w < kW; ++w) mm = nnmax(mm, wmax[w]);
      atomicMax(reinterpret_cast<unsigned int*>(a.tensor_scale), __float_as_uint(nvfp4_tensor_scale(mm * cnorm)));
    }
  }
}

template <int OP, int GC, int SD, bool H16 = false, bool F32 = false>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(kW == 4 ? 2 : 4))) void fast344_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kXBytes];
  __shared__ uint4 sgn[kChunks2];
  __shared__ float wmax[kW];
  const int tid = threadIdx.x;
  for (int c = tid; c < kChunks2; c += kT) {
    uint4 m = make_uint4(0, 0, 0, 0);
    if (a.signs) {
      // chunk c of half h: elements 128 a + 64 h + d, a = cc >> 3, d = 8 (cc & 7) .. + 7
      const int h = c / kChunks, cc = c % kChunks;
      const uint2 sv = *reinterpret_cast<const uint2*>(a.signs + 128 * (cc >> 3) + 64 * h + 8 * (cc & 7));
      m.x = __builtin_amdgcn_perm(0u, sv.x, 0x010C000Cu) & 0x80008000u;
      m.y = __builtin_amdgcn_perm(0u, sv.x, 0x030C020Cu) & 0x80008000u;
      m.z = __builtin_amdgcn_perm(0u, sv.y, 0x010C000Cu) & 0x80008000u;
      m.w = __builtin_amdgcn_perm(0u, sv.y, 0x030C020Cu) & 0x80008000u;
    }
    sgn[c] = m;
  }
  for (int c = tid; c < kXBytes / 16; c += kT) reinterpret_cast<uint4*>(xs)[c] = make_uint4(0, 0, 0, 0);   // a >= 172 stays 0
  if constexpr (kTiles % kW == 0) {
    rows344<OP, GC, SD, kNT, H16, F32>(a, xs, sgn, wmax);
  } else {
    if ((tid >> 6) < kTiles % kW) rows344<OP, GC, SD, kNT, H16, F32>(a, xs, sgn, wmax);
    else rows344<OP, GC, SD, kNT - 1, H16, F32>(a, xs, sgn, wmax);
  }
}

template <int OP, int GC, int SD, int IN>
hipError_t launch344(const KernelArgs& a, hipStream_t s) {
  auto kern = fast344_kernel<OP, GC, SD, IN == RHTQ_IN_F16, IN == RHTQ_IN_F32>;
  static const int max_blocks = resident_blocks((const void*)kern, kT, 0);
  const int grid = (int)(a.rows < max_blocks ? a.rows : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kT), 0, s, a);
  return hipGetLastError();
}

template <int SD, int IN>
hipError_t launch344_int4(const KernelArgs& a, hipStream_t s) {
  if (a.group == kN2) return launch344<OP_INT4, 0, SD, IN>(a, s);   // one group per row
  switch (a.group) {
    case 16: return launch344<OP_INT4, 4, SD, IN>(a, s);
    case 32: return launch344<OP_INT4, 5, SD, IN>(a, s);
    case 64: case 128: case 256: case 512: return launch344<OP_INT4, 6, SD, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}

template <int IN>
hipError_t launch344_op(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return launch344<OP_ROTATE, 6, 0, IN>(a, s);
    case OP_INT4:
      return a.scale_dtype == RHTQ_SCALE_F32 ? launch344_int4<RHTQ_SCALE_F32, IN>(a, s)
                                             : launch344_int4<RHTQ_SCALE_F16, IN>(a, s);
    case OP_NVFP4: return launch344<OP_NVFP4, 4, 0, IN>(a, s);
    case OP_MXFP4: return launch344<OP_MXFP4, 5, 0, IN>(a, s);
    case OP_AMAX: return launch344<OP_AMAX, 6, 0, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}

template <int P, int OP, int GC, int SD, int IN>
hipError_t launch172(const KernelArgs& a, hipStream_t s) {
  auto kern = fast172_kernel<P, OP, GC, SD, IN == RHTQ_IN_F16, IN == RHTQ_IN_F32>;
  static const int max_blocks = resident_blocks((const void*)kern, kT, 0);
  const int64_t vrows = (a.rows + P - 1) / P;
  const int grid = (int)(vrows < max_blocks ? vrows : max_blocks);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kT), 0, s, a);
  return hipGetLastError();
}

template <int P, int SD, int IN>
hipError_t launch172_int4(const KernelArgs& a, hipStream_t s) {
  if (a.group == kN / P) return launch172<P, OP_INT4, 0, SD, IN>(a, s);   // one group per row
  switch (a.group) {
    case 16: return launch172<P, OP_INT4, 4, SD, IN>(a, s);
    case 32: return launch172<P, OP_INT4, 5, SD, IN>(a, s);
    case 64: return launch172<P, OP_INT4, 6, SD, IN>(a, s);
    case 128: return P <= 2 ? launch172<P, OP_INT4, 6, SD, IN>(a, s) : hipErrorNotSupported;
    case 256: return P == 1 ? launch172<P, OP_INT4, 6, SD, IN>(a, s) : hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
}

template <int P, int IN>
hipError_t launch172_p(int op, const KernelArgs& a, hipStream_t s) {
  switch (op) {
    case OP_ROTATE: return launch172<P, OP_ROTATE, 6, 0, IN>(a, s);
    case OP_INT4:
      return a.scale_dtype == RHTQ_SCALE_F32 ? launch172_int4<P, RHTQ_SCALE_F32, IN>(a, s)
                                             : launch172_int4<P, RHTQ_SCALE_F16, IN>(a, s);
    case OP_NVFP4: return launch172<P, OP_NVFP4, 4, 0, IN>(a, s);
    case OP_MXFP4: return launch172<P, OP_MXFP4, 5, 0, IN>(a, s);
    case OP_AMAX: return launch172<P, OP_AMAX, 6, 0, IN>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

namespace {
template <int IN>
hipError_t launch172_any(int op, const KernelArgs& a, hipStream_t s) {
  if (reinterpret_cast<uintptr_t>(a.x) & 15) return hipErrorNotSupported;
  if (a.n == kN && a.sign_period == kN) return launch172_p<1, IN>(op, a, s);
  // 22016 = 172 x 128: the two 64-column halves of each row in turn
  if (a.n == kN2 && a.sign_period == kN2) return launch344_op<IN>(op, a, s);
  // 5504 = 172 x 32 and 2752 = 172 x 16: two and four rows per work row
  if (a.n == kN / 2 && a.sign_period == kN / 2) return launch172_p<2, IN>(op, a, s);
  if (a.n == kN / 4 && a.sign_period == kN / 4) return launch172_p<4, IN>(op, a, s);
  return hipErrorNotSupported;
}
}  // namespace

hipError_t launch_fast172(int op, const KernelArgs& a, hipStream_t s, bool f16in) {
  return f16in ? launch172_any<RHTQ_IN_F16>(op, a, s) : launch172_any<RHTQ_IN_BF16>(op, a, s);
}

hipError_t launch_fast172_f32(int op, const KernelArgs& a, hipStream_t s) {
  return launch172_any<RHTQ_IN_F32>(op, a, s);
}

}  // namespace rhtq
