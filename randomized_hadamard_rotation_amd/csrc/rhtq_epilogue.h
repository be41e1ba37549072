// Quantisation epilogue shared by the two-stage kernels (not part of the public ABI).
//
// Layout it works on: R chunks of 512 consecutive outputs of one row; in chunk q this
// lane holds the eight consecutive outputs cbase(q) + 8 lc + r (r = 0..7), lc =
// (lane >> 4) | ((lane & 15) << 2), as val(q, r) in split units (true value = val * invS).
// So element bits 0-2 are the register index r, bits 3-4 the lane bits 4-5 and bits 5-8
// the lane bits 0-3.
//
// Group maxima: in-lane over the eight values, then across lane bit 4 (element bit 3)
// and lane bit 5 (element bit 4) by swap-and-max steps that pair chunks so every step
// halves the registers, then DPP over lane bits 0-3 (element bits 5-8).  The scale
// arithmetic then runs on the compacted registers, once per group, and the reverse swaps
// broadcast the per-group factor back to the chunk layout.
//
// INT4 (QuaRot reviews, review 2 Summary; reviewer 2 follow-up: nearest rounding):
// s = amax / 7 stored as fp32 / fp16, codes = clamp(rne(y / s_stored), -8, 7) by the
// 1.5 * 2^23 magic-constant FMA.  NVFP4 (NVFP4 methodology thread): E4M3 block scale of
// bmax / (6 g), E2M1 codes by v_cvt_scalef32_pk_fp4_f32 with unit scale; zero-scale blocks
// store code 0.  MXFP4 (OCP MX v1.0; compared with NVFP4 in the same thread): 32-blocks
// share the E8M0 exponent floor(log2(bmax)) - 2, codes as for NVFP4 with that scale.
#pragma once

#include "rhtq_device.h"
#include "rhtq_internal.h"

namespace rhtq {

__device__ __forceinline__ void store_int4_scale(void* scales, int scale_dtype, int64_t gi, float s) {
  if (scale_dtype == RHTQ_SCALE_F32) static_cast<float*>(scales)[gi] = s;
  else static_cast<__half*>(scales)[gi] = __float2half_rn(fminf(s, 65504.0f));
}

// INT4 codes of R chunks in the layout above: inv[q] takes chunk q from split units to scale
// units, clamp says this lane's group needs the [-8, 7] clamp (the clamp runs when any lane of
// the wave needs it); one 4-byte store of eight codes per lane and chunk.
template <int R, typename ValF, typename BaseF>
__device__ __forceinline__ void int4_codes(uint8_t* prow, const float (&inv)[R], const bool clamp, const int lc,
                                           ValF val, BaseF cbase) {
  const bool any_clamp = __builtin_amdgcn_ballot_w64(clamp) != 0;
#pragma unroll
  for (int q = 0; q < R; ++q) {
    uint32_t qb[8];
    if (!any_clamp) {
#pragma unroll
      for (int r = 0; r < 8; ++r) qb[r] = __float_as_uint(__builtin_fmaf(val(q, r), inv[q], 12582912.0f));
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        qb[r] = __float_as_uint(__builtin_amdgcn_fmed3f(val(q, r) * inv[q], -8.0f, 7.0f) + 12582912.0f);
    }
    st_stream(prow + (cbase(q) >> 1) + 4 * lc, pack8_nibbles(qb));
  }
}

// OP is OP_INT4, OP_NVFP4 or OP_MXFP4.  G = log2 of the group (0: one INT4 group per
// row; NVFP4: 4; MXFP4: 5).
// relem0: index of the row's first element in the tensor; N: row width.
// rowmax(m): row maximum (true units) from this lane's maximum (true units), every lane.
// row_writer: this lane stores the row's scale when G == 0.
template <int OP, int R, typename ValF, typename BaseF, typename RowMaxF>
__device__ __forceinline__ void quant_epilogue(const KernelArgs& a, const int64_t row, const int64_t relem0, const int G,
                                               const float invS, const float cnorm, const float gts, const float inv6g,
                                               const int lane, const bool row_writer, ValF val, BaseF cbase,
                                               RowMaxF rowmax) {
  static_assert(R % 2 == 0, "chunks come in pairs");
  const int lc = (lane >> 4) | ((lane & 15) << 2);

  // in-lane maxima of each chunk (split units)
  float mq[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
    mq[q] = m;
  }

  float inv[R];        // per chunk: factor from split units to scale units for this lane's group
  bool clamp = false;  // some group of the wave needs the [-8, 7] clamp

  if (OP == OP_INT4 && G == 0) {
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < R; ++q) m = fmaxf(m, mq[q]);
    const Int4Scale sc = int4_scale(rowmax(m * invS), cnorm, a.scale_dtype);
    clamp = sc.clamp;
#pragma unroll
    for (int q = 0; q < R; ++q) inv[q] = sc.inv * invS;
    if (row_writer) store_int4_scale(a.scales, a.scale_dtype, row, sc.s);
  } else {
    // level 1 (element bit 3, lane bit 4): c1[p] rows 0, 2 <- chunk 2p; rows 1, 3 <- chunk 2p + 1
    constexpr int R1 = R / 2;
    float c1[R1];
#pragma unroll
    for (int p = 0; p < R1; ++p) c1[p] = swap16_max(mq[2 * p], mq[2 * p + 1]);
    const int rw = lane >> 4;    // row of 16 lanes
    const int col = lane & 15;   // element bits 5-8

    if (OP == OP_NVFP4 || G == 4) {
      // 16-element groups: slot (p, lane) is chunk 2p + (rw & 1) with element bit 4 = rw >> 1
      float sl[R1];
#pragma unroll
      for (int p = 0; p < R1; ++p) {
        const int qq = 2 * p + (rw & 1);
        const int64_t gi = (relem0 + cbase(qq) + 16 * (rw >> 1) + 32 * col) >> 4;
        const float bm = c1[p] * invS;   // block maximum, true units
        if constexpr (OP == OP_NVFP4) {
          const uint32_t code = e4m3_code((bm * cnorm) * inv6g);
          const float seff = e4m3_value(code) * gts;
          sl[p] = seff > 0.0f ? (cnorm * __builtin_amdgcn_rcpf(seff)) * invS : 0.0f;
          static_cast<uint8_t*>(a.scales)[gi] = (uint8_t)code;
        } else {
          const Int4Scale sc = int4_scale(bm, cnorm, a.scale_dtype);
          sl[p] = sc.inv * invS;
          clamp |= sc.clamp;
          store_int4_scale(a.scales, a.scale_dtype, gi, sc.s);
        }
      }
#pragma unroll
      for (int p = 0; p < R1; ++p) expand16(sl[p], inv[2 * p], inv[2 * p + 1]);
    } else {
      // level 2 (element bit 4, lane bit 5)
      constexpr int R2 = R1 >= 2 ? R1 / 2 : 1;
      static_assert(R1 == 1 || R1 % 2 == 0, "level 2 pairs the level-1 registers");
      float c2[R2];
      if constexpr (R1 >= 2) {
        // c2[p] row rw holds chunk 4p + rw
#pragma unroll
        for (int p = 0; p < R2; ++p) c2[p] = swap32_max(c1[2 * p], c1[2 * p + 1]);
      } else {
        // one register: rows 0, 2 hold chunk 0 and rows 1, 3 chunk 1 (each twice)
        c2[0] = swap32_max(c1[0], c1[0]);
      }
      // element bits 5 .. G-1 sit in lane bits 0 .. G-6
#pragma unroll
      for (int p = 0; p < R2; ++p) {
        if (G >= 6) c2[p] = dpp_max<0xB1>(c2[p]);    // lane xor 1
        if (G >= 7) c2[p] = dpp_max<0x4E>(c2[p]);    // lane xor 2
        if (G >= 8) c2[p] = dpp_max<0x141>(c2[p]);   // half-row mirror
        if (G >= 9) c2[p] = dpp_max<0x140>(c2[p]);   // row mirror
      }
      float sl[R2];
      const bool lane_writes = (col & ((1 << (G - 5)) - 1)) == 0 && (R1 >= 2 || rw < 2);
#pragma unroll
      for (int p = 0; p < R2; ++p) {
        const int qq = R1 >= 2 ? 4 * p + rw : (rw & 1);
        const int64_t gi = (relem0 + cbase(qq) + 32 * col) >> G;
        if constexpr (OP == OP_MXFP4) {
          const float bm = (c2[p] * invS) * cnorm;   // block maximum of the rotated values
          const int ex = mx_exponent(bm);
          sl[p] = bm > 0.0f ? __builtin_ldexpf(invS * cnorm, -ex) : 0.0f;
          if (lane_writes) static_cast<uint8_t*>(a.scales)[gi] = (uint8_t)(ex + 127);
        } else {
          const Int4Scale sc = int4_scale(c2[p] * invS, cnorm, a.scale_dtype);
          sl[p] = sc.inv * invS;
          clamp |= sc.clamp;
          if (lane_writes) store_int4_scale(a.scales, a.scale_dtype, gi, sc.s);
        }
      }
      float e1[R1];
      if constexpr (R1 >= 2) {
#pragma unroll
        for (int p = 0; p < R2; ++p) expand32(sl[p], e1[2 * p], e1[2 * p + 1]);
      } else {
        e1[0] = sl[0];
      }
#pragma unroll
      for (int p = 0; p < R1; ++p) expand16(e1[p], inv[2 * p], inv[2 * p + 1]);
    }
  }

  // codes: 8 per lane and chunk -> one dword; a wave store covers 256 contiguous bytes
  uint8_t* prow = a.packed + (relem0 >> 1);
  if constexpr (OP == OP_INT4) {
    int4_codes<R>(prow, inv, clamp, lc, val, cbase);
  } else if constexpr (OP == OP_NVFP4 || OP == OP_MXFP4) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const float s = inv[q];
      uint32_t w = 0;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(q, 0) * s, val(q, 1) * s, 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(q, 2) * s, val(q, 3) * s, 1.0f, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(q, 4) * s, val(q, 5) * s, 1.0f, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(q, 6) * s, val(q, 7) * s, 1.0f, 3);
      st_stream(prow + (cbase(q) >> 1) + 4 * lc, s > 0.0f ? w : 0u);   // zero-scale block -> code 0
    }
  }
}

// The same epilogue for the linear layout of the paired 4096 kernel: in chunk q this lane holds
// the eight consecutive outputs cbase(q) + 8 lane + r, so element bits 0-2 are the register
// index and bits 3-8 the lane.  A group of 2^G elements (G = 4 .. 9) spans 2^(G - 3) aligned
// lanes, reduced by group_max; every lane of a group computes the group's scale and the
// group's first lane stores it.  Codes go out as 4-byte stores, one dword per lane and chunk,
// so each wave store covers 256 contiguous bytes in lane order.
template <int OP, int R, typename ValF, typename BaseF, typename RowMaxF>
__device__ __forceinline__ void quant_epilogue_lin(const KernelArgs& a, const int64_t row, const int64_t relem0,
                                                   const int G, const float invS, const float cnorm, const float gts,
                                                   const float inv6g, const int lane, const bool row_writer, ValF val,
                                                   BaseF cbase, RowMaxF rowmax) {
  float mq[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(val(q, r)));
    mq[q] = m;
  }
  float inv[R];
  bool clamp = false;
  if (OP == OP_INT4 && G == 0) {
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < R; ++q) m = fmaxf(m, mq[q]);
    const Int4Scale sc = int4_scale(rowmax(m * invS), cnorm, a.scale_dtype);
    clamp = sc.clamp;
#pragma unroll
    for (int q = 0; q < R; ++q) inv[q] = sc.inv * invS;
    if (row_writer) store_int4_scale(a.scales, a.scale_dtype, row, sc.s);
  } else {
    // a group of 2^G elements spans 2^(G - 3) lanes (G = 4 .. 9)
    const int gl = 1 << (G - 3);
    const bool writer = (lane & (gl - 1)) == 0;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const float bmx = group_max(mq[q], gl) * invS;   // group maximum, true units (unnormalised)
      const int64_t gi = (relem0 + cbase(q) + 8 * lane) >> G;
      if constexpr (OP == OP_NVFP4) {
        const uint32_t code = e4m3_code((bmx * cnorm) * inv6g);
        const float seff = e4m3_value(code) * gts;
        inv[q] = seff > 0.0f ? (cnorm * __builtin_amdgcn_rcpf(seff)) * invS : 0.0f;
        if (writer) static_cast<uint8_t*>(a.scales)[gi] = (uint8_t)code;
      } else if constexpr (OP == OP_MXFP4) {
        const float bm = bmx * cnorm;
        const int ex = mx_exponent(bm);
        inv[q] = bm > 0.0f ? __builtin_ldexpf(invS * cnorm, -ex) : 0.0f;
        if (writer) static_cast<uint8_t*>(a.scales)[gi] = (uint8_t)(ex + 127);
      } else {
        const Int4Scale sc = int4_scale(bmx, cnorm, a.scale_dtype);
        inv[q] = sc.inv * invS;
        clamp |= sc.clamp;
        if (writer) store_int4_scale(a.scales, a.scale_dtype, gi, sc.s);
      }
    }
  }
  uint8_t* const pl = a.packed + (relem0 >> 1) + 4 * lane;   // this lane's dword of chunk 0
  if constexpr (OP == OP_INT4) {
    const bool any_clamp = __builtin_amdgcn_ballot_w64(clamp) != 0;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      uint32_t qb[8];
      if (!any_clamp) {
#pragma unroll
        for (int r = 0; r < 8; ++r) qb[r] = __float_as_uint(__builtin_fmaf(val(q, r), inv[q], 12582912.0f));
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r)
          qb[r] = __float_as_uint(__builtin_amdgcn_fmed3f(val(q, r) * inv[q], -8.0f, 7.0f) + 12582912.0f);
      }
      st_stream(pl + (cbase(q) >> 1), pack8_nibbles(qb));
    }
  } else {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const float s = inv[q];
      uint32_t w = 0;
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(q, 0) * s, val(q, 1) * s, 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(q, 2) * s, val(q, 3) * s, 1.0f, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(q, 4) * s, val(q, 5) * s, 1.0f, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, val(q, 6) * s, val(q, 7) * s, 1.0f, 3);
      st_stream(pl + (cbase(q) >> 1), s > 0.0f ? w : 0u);
    }
  }
}
}  // namespace rhtq
