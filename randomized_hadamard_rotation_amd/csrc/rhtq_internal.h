// Internal interfaces between the host entry points (rhtq_api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace rhtq {

enum Op : int {
  OP_ROTATE = 0,   // y fp32
  OP_INT4 = 1,     // packed INT4 + scales
  OP_NVFP4 = 2,    // packed E2M1 + E4M3 scales, reads the tensor scale g
  OP_AMAX = 3,     // atomic max of g = fl32(|y| / 2688) bits into tensor_scale (NVFP4 dynamic pre-pass)
  OP_INVERSE = 4,  // packed + scales -> x fp32
  OP_MXFP4 = 5,    // packed E2M1 + E8M0 scales of 32-blocks
};

struct KernelArgs {
  const void* x;            // forward input [rows][n] (bf16 or fp32)
  const int8_t* signs;      // [n] or null
  int64_t rows;
  int32_t n;
  int32_t group;            // elements per scale group (n for per-token)
  int32_t scale_dtype;      // RHTQ_SCALE_*
  float* y;                 // OP_ROTATE / OP_INVERSE output
  uint8_t* packed;          // OP_INT4 / OP_NVFP4 output
  void* scales;             // OP_INT4 / OP_NVFP4 output
  float* tensor_scale;      // OP_NVFP4 input g, OP_AMAX accumulator (as uint bits)
  const uint8_t* in_packed; // OP_INVERSE input
  const void* in_scales;    // OP_INVERSE input
  const float* in_tensor_scale;  // OP_INVERSE input (NVFP4)
  int32_t inv_fmt;          // OP_INVERSE: RHTQ_FMT_*
  int32_t sign_period;      // signs repeat every sign_period elements of the flattened rows (a multiple
                            // of n; n itself except for block-diagonal calls, where rows of width n are
                            // the b-blocks of longer rows and the sign vector spans the long row)
};

// Generic LDS-staged path: every width, both input types, every op.
// Returns hipSuccess or the launch error.
hipError_t launch_generic(int op, int in_dtype, const KernelArgs& a, hipStream_t s);

// Register-resident fast path for 16-bit input: bf16, or fp16 when f16in (the same kernels with
// stage 1 on the f16 matrix-core instruction).  Returns hipErrorNotSupported when the
// (op, n, group, input type) combination has no fast kernel; the caller then uses the generic one.
hipError_t launch_fast(int op, const KernelArgs& a, hipStream_t s, bool f16in = false);

// fp32 input on the single-stage register-resident kernels (widths 16 .. 8192, 3072, 6144), the
// 16384, 12288, 24576 and 172 x 2^k kernels: each value is split into three exact bf16 terms for the
// stage-1 products.  Returns
// hipErrorNotSupported where that kernel has no variant; the caller then uses the generic one.
hipError_t launch_fast_f32(int op, const KernelArgs& a, hipStream_t s);

// Two-wave kernel for 12288-wide rows (called by launch_fast), and its fp32-input form
// (called by launch_fast_f32).
hipError_t launch_fast12(int op, const KernelArgs& a, hipStream_t s, bool f16in = false);
hipError_t launch_fast12_f32(int op, const KernelArgs& a, hipStream_t s);

// The grid launch_fast12 uses for per-group INT4 on `rows` rows (resident workgroups, at most
// one per row); the streaming-floor measurement launches the same grid.
int64_t fast12_grid(int64_t rows);

// Four-wave kernel for 24576-wide rows, H12 (x) H2048 (called by launch_fast).
hipError_t launch_fast24(int op, const KernelArgs& a, hipStream_t s, bool f16in = false);
hipError_t launch_fast24_f32(int op, const KernelArgs& a, hipStream_t s);   // fp32 input

// Matrix-core kernel for 11008-wide rows, H172 (x) H64, and 5504, 2752, 22016 (called by
// launch_fast), and its fp32-input form (called by launch_fast_f32: three exact bf16 terms per
// value taken through the kernel's LDS tile in turn, accumulating into the same products).
hipError_t launch_fast172(int op, const KernelArgs& a, hipStream_t s, bool f16in = false);
hipError_t launch_fast172_f32(int op, const KernelArgs& a, hipStream_t s);

// Two-stage matrix-core kernel for 1024-, 2048- and 4096-wide rows (called by launch_fast).
hipError_t launch_fast2(int op, const KernelArgs& a, hipStream_t s, bool f16in = false);

// 8192- and 16384-wide rows, 2 or 4 waves per row with the top index bits exchanged through LDS
// (called by launch_fast).
hipError_t launch_fastw(int op, const KernelArgs& a, hipStream_t s, bool f16in = false);
// Its fp32-input form at 16384 (called by launch_fast_f32; 8192 has the single-stage kernel's).
hipError_t launch_fastw_f32(int op, const KernelArgs& a, hipStream_t s);

// Integer matrix-core inverse for KV-cache rows (64, 128, 256) with one INT4 scale per row.
// Returns hipErrorNotSupported for other cases (the generic kernel then runs).
hipError_t launch_inverse_fast(const KernelArgs& a, hipStream_t s);

// RHTQ_FORCE_GENERIC=1 routes every call to the generic kernels (read once).
inline bool getenv_fast_disabled() {
  static const bool v = [] {
    const char* e = getenv("RHTQ_FORCE_GENERIC");
    return e != nullptr && e[0] == '1';
  }();
  return v;
}

// RHTQ_TEST_FAIL_LAUNCH=1 makes every entry point stop where it would first call HIP, after all
// argument checks, and report a runtime error: the launch-error path, testable without a failing
// launch (read once).
inline bool getenv_test_fail_launch() {
  static const bool v = [] {
    const char* e = getenv("RHTQ_TEST_FAIL_LAUNCH");
    return e != nullptr && e[0] == '1';
  }();
  return v;
}

// RHTQ_DISABLE_FAST2=1 keeps 1024..4096-wide rows on the single-stage kernel (read once).
inline bool getenv_fast2_disabled() {
  static const bool v = [] {
    const char* e = getenv("RHTQ_DISABLE_FAST2");
    return e != nullptr && e[0] == '1';
  }();
  return v;
}

// Resident workgroups of `kern` on the current device: CUs x workgroups per CU (at least one).
// The persistent kernels size their grid with it; their loops stride over rows, so the value only
// affects speed.  Callers keep it in a function-local static, which C++ initialises once and
// thread-safely.
inline int resident_blocks(const void* kern, int threads, size_t lds) {
  int dev = 0, cus = 256, per_cu = 1;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return cus * per_cu;
}

// Clears the word the dynamic NVFP4 pre-pass accumulates into.
hipError_t launch_zero_word(float* p, hipStream_t s);

}  // namespace rhtq
