// Generic LDS-staged kernel: every supported width, bf16 or fp32 input, every op.
//
// One workgroup of 256 threads takes a tile of whole rows (about 4096 elements, or
// one row for wider rows) into LDS as fp32, runs the Walsh-Hadamard butterflies
// three index bits per pass (QuaRot reviews, review 1 Summary: the online Hadamard
// uses the Walsh-Hadamard fast algorithm), the order-12 factor for n = 12*m
// (KronQ issue #2, Model Details: 12288 = 12 x 1024) or the order-172 factor for
// n = 172*m (QuaRot reviews, review 2 Questions: Llama 2 7B), then the epilogue.  The
// register-resident kernels in rhtq_fast.hip cover the bf16 hot shapes; this one
// is the complete fallback and the path for fp32 input and for the inverse.
#include <hip/hip_fp16.h>

#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

constexpr int kThreads = 256;
constexpr int kTileTarget = 4096;

// Sign bits of H172 and of its transpose, for the dense order-172 contraction.
__constant__ H172Bits<false> kH172;
__constant__ H172Bits<true> kH172T;

__host__ __device__ constexpr int lds_idx(int j) { return j + (j >> 5); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 3-bit E2M1 magnitude of a >= 0, nearest even, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const float mag = m < 4 ? 0.5f * (float)m : (m == 4 ? 2.0f : (m == 5 ? 3.0f : (m == 6 ? 4.0f : 6.0f)));
  return (c & 8u) ? -mag : mag;
}

template <int P>
__device__ __forceinline__ void butterflies(float* v) {
#pragma unroll
  for (int h = 1; h < (1 << P); h <<= 1) {
#pragma unroll
    for (int k = 0; k < (1 << P); ++k) {
      if ((k & h) == 0) {
        const float a = v[k], b = v[k | h];
        v[k] = a + b;
        v[k | h] = a - b;
      }
    }
  }
}

template <int P, int TE>
__device__ __forceinline__ void fwht_pass(float* lds, int b) {
  const int ncos = TE >> P;
  for (int w = threadIdx.x; w < ncos; w += kThreads) {
    const int base = ((w >> b) << (b + P)) | (w & ((1 << b) - 1));
    float v[1 << P];
#pragma unroll
    for (int k = 0; k < (1 << P); ++k) v[k] = lds[lds_idx(base + (k << b))];
    butterflies<P>(v);
#pragma unroll
    for (int k = 0; k < (1 << P); ++k) lds[lds_idx(base + (k << b))] = v[k];
  }
}

template <int IN, int F, int LOGM, int OP>
__global__ __launch_bounds__(kThreads) void generic_kernel(KernelArgs a) {
  constexpr int M = 1 << LOGM;
  constexpr int N = F * M;
  constexpr int R = (N >= kTileTarget) ? 1 : kTileTarget / N;
  constexpr int TE = R * N;
  constexpr int NCHUNK = TE / 8;
  extern __shared__ float smem[];
  float* lds = smem;
  float* red = smem + lds_idx(TE);
  const int tid = threadIdx.x;
  const float cnorm = (float)(1.0 / __builtin_sqrt((double)N));
  const int64_t ntiles = (a.rows + R - 1) / R;
  float run_max = 0.0f;  // OP_AMAX

  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * R;
    const int nrows = (int)((a.rows - row0) < R ? (a.rows - row0) : R);
    const int valid = nrows * N;
    const int64_t gbase = row0 * (int64_t)N;

    // ---------------- load ----------------
    for (int c = tid; c < NCHUNK; c += kThreads) {
      const int e0 = c * 8;
      float v[8];
      if (e0 < valid) {
        if constexpr (OP == OP_INVERSE) {
          const uint32_t w = *(const uint32_t*)(a.in_packed + (gbase + e0) / 2);
          const int64_t gidx = (gbase + e0) / a.group;
          if (a.inv_fmt == RHTQ_FMT_INT4) {
            const float s = a.scale_dtype == RHTQ_SCALE_F32
                                ? ((const float*)a.in_scales)[gidx]
                                : __half2float(((const __half*)a.in_scales)[gidx]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int q = ((int)((w >> (4 * e)) & 15u) ^ 8) - 8;
              v[e] = (float)q * s;
            }
          } else {
            const uint32_t sb = ((const uint8_t*)a.in_scales)[gidx];
            const float seff = a.inv_fmt == RHTQ_FMT_MXFP4 ? __builtin_ldexpf(1.0f, (int)sb - 127)
                                                           : e4m3_value(sb) * a.in_tensor_scale[0];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = e2m1_value((w >> (4 * e)) & 15u) * seff;
          }
        } else {
          if constexpr (IN == RHTQ_IN_BF16) {
            const uint4 raw = *(const uint4*)((const uint16_t*)a.x + gbase + e0);
            v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x);
            v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
            v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z);
            v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
          } else if constexpr (IN == RHTQ_IN_F16) {
            const uint4 raw = *(const uint4*)((const uint16_t*)a.x + gbase + e0);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {   // f16 -> f32 is exact
              v[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xFFFFu));
              v[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
            }
          } else {
            const float4* p = (const float4*)((const float*)a.x + gbase + e0);
            const float4 p0 = p[0], p1 = p[1];
            v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
            v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
          }
          if (a.signs) {
            const int col = (int)((gbase + e0) % a.sign_period);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (a.signs[col + e] < 0) v[e] = -v[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) lds[lds_idx(e0 + e)] = v[e];
    }
    __syncthreads();

    // ---------------- transform ----------------
#pragma unroll
    for (int b = 0; b < LOGM; b += 3) {
      if (LOGM - b >= 3) fwht_pass<3, TE>(lds, b);
      else if (LOGM - b == 2) fwht_pass<2, TE>(lds, b);
      else fwht_pass<1, TE>(lds, b);
      __syncthreads();
    }
    if constexpr (F == 172) {
      // dense order-172 contraction across j1 for every (row, j2): work item = (row, j2, four
      // consecutive outputs); all reads finish before the barrier, results are held in registers
      constexpr int ITEMS = R * M * 43;
      constexpr int PER = (ITEMS + kThreads - 1) / kThreads;
      const H172Bits<OP == OP_INVERSE>& hb = [] () -> const H172Bits<OP == OP_INVERSE>& {
        if constexpr (OP == OP_INVERSE) return kH172T; else return kH172;
      }();
      float res[PER][4];
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int w = tid + t * kThreads;
        if (w < ITEMS) {
          const int iq = (w / M) % 43, j2 = w % M, r = w / (M * 43);
          const int base = r * N + j2;
          // fp64 sums: a 172-term fp32 chain would lose up to 172 ulps of its partial sums
          double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
          for (int jw = 0; jw < 6; ++jw) {
            uint32_t bits[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) bits[q] = hb.w[4 * iq + q][jw];
            const int jn = jw < 5 ? 32 : 172 - 160;
#pragma unroll 4
            for (int jj = 0; jj < jn; ++jj) {
              const int j = 32 * jw + jj;
              const uint32_t v = __float_as_uint(lds[lds_idx(base + j * M)]);
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[q] += (double)__uint_as_float(v ^ (((bits[q] >> jj) & 1u) << 31));
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) res[t][q] = (float)acc[q];
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int w = tid + t * kThreads;
        if (w < ITEMS) {
          const int iq = (w / M) % 43, j2 = w % M, r = w / (M * 43);
#pragma unroll
          for (int q = 0; q < 4; ++q) lds[lds_idx(r * N + (4 * iq + q) * M + j2)] = res[t][q];
        }
      }
      __syncthreads();
    }
    if constexpr (F == 12) {
      for (int w = tid; w < R * M; w += kThreads) {
        const int base = (w / M) * N + (w % M);
        float v[12], o[12];
#pragma unroll
        for (int j = 0; j < 12; ++j) v[j] = lds[lds_idx(base + j * M)];
#pragma unroll
        for (int i = 0; i < 12; ++i) {
          float acc = 0.0f;
#pragma unroll
          for (int j = 0; j < 12; ++j) {
            const int h = (OP == OP_INVERSE) ? h12_entry(j, i) : h12_entry(i, j);
            acc = h > 0 ? acc + v[j] : acc - v[j];
          }
          o[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 12; ++i) lds[lds_idx(base + i * M)] = o[i];
      }
      __syncthreads();
    }

    // ---------------- epilogue ----------------
    if constexpr (OP == OP_ROTATE || OP == OP_INVERSE) {
      for (int c = tid; c < NCHUNK; c += kThreads) {
        const int e0 = c * 8;
        if (e0 >= valid) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = lds[lds_idx(e0 + e)] * cnorm;
        if constexpr (OP == OP_INVERSE) {
          if (a.signs) {
            const int col = (int)((gbase + e0) % a.sign_period);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (a.signs[col + e] < 0) v[e] = -v[e];
          }
        }
        float4* p = (float4*)(a.y + gbase + e0);
        p[0] = make_float4(v[0], v[1], v[2], v[3]);
        p[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    } else if constexpr (OP == OP_AMAX) {
      for (int c = tid; c < NCHUNK; c += kThreads) {
        const int e0 = c * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) run_max = fmaxf(run_max, fabsf(lds[lds_idx(e0 + e)]));
      }
    } else {
      // normalise in place and collect chunk maxima
      for (int c = tid; c < NCHUNK; c += kThreads) {
        const int e0 = c * 8;
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = lds[lds_idx(e0 + e)] * cnorm;
          lds[lds_idx(e0 + e)] = y;
          m = fmaxf(m, fabsf(y));
        }
        red[c] = m;
      }
      __syncthreads();
      const int g8 = a.group / 8;  // chunks per group (>= 2; 1.5 * 2^k for per-token 12 * 2^k rows)
      for (int s = 1; s < g8; s <<= 1) {
        for (int c = tid; c < NCHUNK; c += kThreads) {
          const int local = c % g8;
          if ((local & (2 * s - 1)) == 0 && local + s < g8) red[c] = fmaxf(red[c], red[c + s]);
        }
        __syncthreads();
      }
      const float gts = (OP == OP_NVFP4) ? a.tensor_scale[0] : 0.0f;
      for (int c = tid; c < NCHUNK; c += kThreads) {
        const int e0 = c * 8;
        if (e0 >= valid) continue;
        const int cg = (c / g8) * g8;
        const float gmax = red[cg];
        const int64_t gidx = (gbase + e0) / a.group;
        const bool first = (c == cg);
        uint32_t word = 0;
        if constexpr (OP == OP_INT4) {
          const float s = gmax / 7.0f;
          float sq;
          if (a.scale_dtype == RHTQ_SCALE_F32) {
            sq = s;
            if (first) ((float*)a.scales)[gidx] = s;
          } else {
            const __half h = __float2half_rn(fminf(s, 65504.0f));  // fp16 saturates
            sq = __half2float(h);
            if (first) ((__half*)a.scales)[gidx] = h;
          }
          if (sq > 0.0f) {
            const float inv = 1.0f / sq;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float q = __builtin_rintf(lds[lds_idx(e0 + e)] * inv);
              q = fminf(fmaxf(q, -8.0f), 7.0f);
              word |= ((uint32_t)(int)q & 15u) << (4 * e);
            }
          }
        } else if constexpr (OP == OP_MXFP4) {
          const int ex = mx_exponent(gmax);
          if (first) ((uint8_t*)a.scales)[gidx] = (uint8_t)(ex + 127);
          if (gmax > 0.0f) {
            const float inv = __builtin_ldexpf(1.0f, -ex);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = lds[lds_idx(e0 + e)] * inv;
              const uint32_t code = e2m1_mag(fabsf(v)) | (__float_as_uint(v) >> 31 << 3);
              word |= code << (4 * e);
            }
          }
        } else {  // OP_NVFP4
          uint32_t sc = 0;
          if (gts > 0.0f) sc = e4m3_code(gmax / (6.0f * gts));
          if (first) ((uint8_t*)a.scales)[gidx] = (uint8_t)sc;
          const float seff = e4m3_value(sc) * gts;
          if (seff > 0.0f) {
            const float inv = 1.0f / seff;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = lds[lds_idx(e0 + e)] * inv;
              const uint32_t code = e2m1_mag(fabsf(v)) | (__float_as_uint(v) >> 31 << 3);
              word |= code << (4 * e);
            }
          }
        }
        *(uint32_t*)(a.packed + (gbase + e0) / 2) = word;
      }
    }
    __syncthreads();
  }

  if constexpr (OP == OP_AMAX) {
    // block maximum, then one atomic per block (ordering of positive floats as uints)
    for (int off = 32; off > 0; off >>= 1) run_max = fmaxf(run_max, __shfl_xor(run_max, off));
    __shared__ float wmax[kThreads / 64];
    if ((tid & 63) == 0) wmax[tid >> 6] = run_max;
    __syncthreads();
    if (tid == 0) {
      float m = wmax[0];
      for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, wmax[w]);
      atomicMax((unsigned int*)a.tensor_scale, __float_as_uint(nvfp4_tensor_scale(m * cnorm)));
    }
  }
}

template <int IN, int F, int LOGM, int OP>
hipError_t launch_one(const KernelArgs& a, hipStream_t s) {
  constexpr int M = 1 << LOGM;
  constexpr int N = F * M;
  constexpr int R = (N >= kTileTarget) ? 1 : kTileTarget / N;
  constexpr int TE = R * N;
  const size_t lds_bytes = (size_t)(lds_idx(TE) + TE / 8) * sizeof(float);
  auto kern = generic_kernel<IN, F, LOGM, OP>;
  if (lds_bytes > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds_bytes);
    if (e != hipSuccess) return e;
  }
  const int64_t ntiles = (a.rows + R - 1) / R;
  const int grid = (int)(ntiles < 4096 ? ntiles : 4096);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds_bytes, s, a);
  return hipGetLastError();
}

template <int IN, int OP>
hipError_t dispatch_width(const KernelArgs& a, hipStream_t s) {
  switch (a.n) {
    case 16: return launch_one<IN, 1, 4, OP>(a, s);
    case 32: return launch_one<IN, 1, 5, OP>(a, s);
    case 64: return launch_one<IN, 1, 6, OP>(a, s);
    case 128: return launch_one<IN, 1, 7, OP>(a, s);
    case 256: return launch_one<IN, 1, 8, OP>(a, s);
    case 512: return launch_one<IN, 1, 9, OP>(a, s);
    case 1024: return launch_one<IN, 1, 10, OP>(a, s);
    case 2048: return launch_one<IN, 1, 11, OP>(a, s);
    case 4096: return launch_one<IN, 1, 12, OP>(a, s);
    case 8192: return launch_one<IN, 1, 13, OP>(a, s);
    case 16384: return launch_one<IN, 1, 14, OP>(a, s);
    case 3072: return launch_one<IN, 12, 8, OP>(a, s);
    case 6144: return launch_one<IN, 12, 9, OP>(a, s);
    case 12288: return launch_one<IN, 12, 10, OP>(a, s);
    case 24576: return launch_one<IN, 12, 11, OP>(a, s);
    case 2752: return launch_one<IN, 172, 4, OP>(a, s);
    case 5504: return launch_one<IN, 172, 5, OP>(a, s);
    case 11008: return launch_one<IN, 172, 6, OP>(a, s);
    case 22016: return launch_one<IN, 172, 7, OP>(a, s);
    default: return hipErrorInvalidValue;
  }
}

__global__ void zero_word_kernel(float* p) { *p = 0.0f; }

// g = fl32(amax / (6 * 448)), in place over the accumulated amax.

}  // namespace

hipError_t launch_generic(int op, int in_dtype, const KernelArgs& a, hipStream_t s) {
  if (in_dtype == RHTQ_IN_BF16) {
    switch (op) {
      case OP_ROTATE: return dispatch_width<RHTQ_IN_BF16, OP_ROTATE>(a, s);
      case OP_INT4: return dispatch_width<RHTQ_IN_BF16, OP_INT4>(a, s);
      case OP_NVFP4: return dispatch_width<RHTQ_IN_BF16, OP_NVFP4>(a, s);
      case OP_MXFP4: return dispatch_width<RHTQ_IN_BF16, OP_MXFP4>(a, s);
      case OP_AMAX: return dispatch_width<RHTQ_IN_BF16, OP_AMAX>(a, s);
      case OP_INVERSE: return dispatch_width<RHTQ_IN_BF16, OP_INVERSE>(a, s);
    }
  } else if (in_dtype == RHTQ_IN_F16) {
    switch (op) {
      case OP_ROTATE: return dispatch_width<RHTQ_IN_F16, OP_ROTATE>(a, s);
      case OP_INT4: return dispatch_width<RHTQ_IN_F16, OP_INT4>(a, s);
      case OP_NVFP4: return dispatch_width<RHTQ_IN_F16, OP_NVFP4>(a, s);
      case OP_MXFP4: return dispatch_width<RHTQ_IN_F16, OP_MXFP4>(a, s);
      case OP_AMAX: return dispatch_width<RHTQ_IN_F16, OP_AMAX>(a, s);
      case OP_INVERSE: return hipErrorInvalidValue;  // inverse input is packed codes
    }
  } else {
    switch (op) {
      case OP_ROTATE: return dispatch_width<RHTQ_IN_F32, OP_ROTATE>(a, s);
      case OP_INT4: return dispatch_width<RHTQ_IN_F32, OP_INT4>(a, s);
      case OP_NVFP4: return dispatch_width<RHTQ_IN_F32, OP_NVFP4>(a, s);
      case OP_MXFP4: return dispatch_width<RHTQ_IN_F32, OP_MXFP4>(a, s);
      case OP_AMAX: return dispatch_width<RHTQ_IN_F32, OP_AMAX>(a, s);
      case OP_INVERSE: return hipErrorInvalidValue;  // inverse input is packed codes
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_zero_word(float* p, hipStream_t s) {
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, p);
  return hipGetLastError();
}


}  // namespace rhtq
