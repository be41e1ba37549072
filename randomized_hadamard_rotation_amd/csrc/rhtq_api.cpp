// Host entry points of librhtq.so: argument checks, dispatch, launch.
// Every check happens before the first HIP call, so a rejected call enqueues nothing.
#include <stdint.h>

#include <climits>

#include "rhtq.h"
#include "rhtq_internal.h"

namespace {

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// n = 2^k (16..16384), 12 * 2^k (2^k in 256..2048) or 172 * 2^k (2^k in 16..128): the
// power-of-two widths, the 12 x 2^k widths (KronQ issue #2, Model Details: 12288 = 12 x 1024)
// and the 172 x 2^k widths (QuaRot reviews, review 2 Questions: 11008 = 172 x 64, Llama 2 7B).
bool width_ok(int32_t n) {
  if (is_pow2(n)) return n >= 16 && n <= 16384;
  if (n % 172 == 0) {
    const int32_t m = n / 172;
    return is_pow2(m) && m >= 16 && m <= 128;
  }
  if (n % 12 == 0) {
    const int32_t m = n / 12;
    return is_pow2(m) && m >= 256 && m <= 2048;
  }
  return false;
}

bool group_ok(int32_t n, int fmt, int32_t group) {
  if (fmt == RHTQ_FMT_INT4) return group == 0 || (is_pow2(group) && group >= 16 && n % group == 0);
  if (fmt == RHTQ_FMT_NVFP4) return group == 16;
  if (fmt == RHTQ_FMT_MXFP4) return group == 32 && n % 32 == 0;
  return false;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? RHTQ_OK : RHTQ_EHIP; }

// The matrix-core kernels for an input type; hipErrorNotSupported sends the call to the generic one.
hipError_t fast_for(int in_dtype, int op, const rhtq::KernelArgs& a, hipStream_t s) {
  if (in_dtype == RHTQ_IN_BF16) return rhtq::launch_fast(op, a, s);
  if (in_dtype == RHTQ_IN_F16) return rhtq::launch_fast(op, a, s, /*f16=*/true);
  return rhtq::launch_fast_f32(op, a, s);
}

// Shared checks of rhtq_forward / rhtq_inverse.  Returns RHTQ_OK or the status.
int check_quant_args(int64_t tokens, int32_t n, int fmt, int32_t group, int scale_dtype) {
  if (tokens < 0) return RHTQ_EINVAL;
  if (fmt != RHTQ_FMT_INT4 && fmt != RHTQ_FMT_NVFP4 && fmt != RHTQ_FMT_MXFP4) return RHTQ_EINVAL;
  if (scale_dtype != RHTQ_SCALE_F32 && scale_dtype != RHTQ_SCALE_F16 && scale_dtype != RHTQ_SCALE_E4M3 &&
      scale_dtype != RHTQ_SCALE_E8M0)
    return RHTQ_EINVAL;
  if (!width_ok(n) || !group_ok(n, fmt, group)) return RHTQ_EUNSUPPORTED;
  if (fmt == RHTQ_FMT_INT4 && scale_dtype != RHTQ_SCALE_F32 && scale_dtype != RHTQ_SCALE_F16)
    return RHTQ_EUNSUPPORTED;
  if (fmt == RHTQ_FMT_NVFP4 && scale_dtype != RHTQ_SCALE_E4M3) return RHTQ_EUNSUPPORTED;
  if (fmt == RHTQ_FMT_MXFP4 && scale_dtype != RHTQ_SCALE_E8M0) return RHTQ_EUNSUPPORTED;
  return RHTQ_OK;
}

uintptr_t scale_align(int scale_dtype) {
  return scale_dtype == RHTQ_SCALE_F32 ? 4 : (scale_dtype == RHTQ_SCALE_F16 ? 2 : 1);
}

// ---- shared bodies of the plain and block-diagonal entry points -------------------------------
// A block-diagonal call on rows of width n with blocks of b runs the kernels on tokens * n / b rows
// of width b whose signs repeat every n elements; the memory layouts of x, y, codes and scales are
// the same either way.  block == n is the plain call.

// Rows of a block-diagonal call need not have a Hadamard width themselves (11008 = 86 x 128 for
// the Llama-2-7B intermediate activation): only the block must, and it must divide the row.
constexpr int32_t kMaxBlockedWidth = 1 << 20;

bool block_ok(int32_t n, int32_t block) {
  if (block == n) return width_ok(n);
  return is_pow2(block) && block >= 16 && block < n && n % block == 0 && n <= kMaxBlockedWidth;
}

// Fills the shape fields of a; RHTQ_OK or the status.
int shape_args(int64_t tokens, int32_t n, int32_t block, rhtq::KernelArgs& a) {
  if (tokens < 0) return RHTQ_EINVAL;
  if (!block_ok(n, block)) return RHTQ_EUNSUPPORTED;
  const int64_t per = n / block;
  if (tokens > INT64_MAX / per) return RHTQ_EINVAL;
  a.rows = tokens * per;
  a.n = block;
  a.sign_period = n;
  return RHTQ_OK;
}

// Quantisation arguments of a call with blocks of b: the group lies inside a block; one group per
// row (group 0) only when the block is the whole row.
int check_quant_block(int32_t n, int32_t block, int fmt, int32_t group, int scale_dtype) {
  const int st = check_quant_args(0, block, fmt, group, scale_dtype);
  if (st != RHTQ_OK) return st;
  if (group == 0 && block != n) return RHTQ_EUNSUPPORTED;
  return RHTQ_OK;
}

int rotate_impl(const void* x, int in_dtype, int64_t tokens, int32_t n, int32_t block, const int8_t* signs,
                float* y_out, rhtq_stream_t stream) {
  if (in_dtype != RHTQ_IN_BF16 && in_dtype != RHTQ_IN_F16 && in_dtype != RHTQ_IN_F32) return RHTQ_EINVAL;
  rhtq::KernelArgs a{};
  const int st = shape_args(tokens, n, block, a);
  if (st != RHTQ_OK) return st;
  if (tokens == 0) return RHTQ_OK;
  if (!x || !y_out) return RHTQ_EINVAL;
  if (!aligned(x, 16) || !aligned(y_out, 16) || !aligned(signs, 16)) return RHTQ_EINVAL;
  a.x = x;
  a.signs = signs;
  a.group = a.n;
  a.y = y_out;
  if (rhtq::getenv_test_fail_launch()) return RHTQ_EHIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    const hipError_t e = fast_for(in_dtype, rhtq::OP_ROTATE, a, s);
    if (e != hipErrorNotSupported) return from_hip(e);
  }
  return from_hip(rhtq::launch_generic(rhtq::OP_ROTATE, in_dtype, a, s));
}

int forward_impl(const void* x, int in_dtype, int64_t tokens, int32_t n, int32_t block, const int8_t* signs,
                 int fmt, int32_t group, int scale_dtype, uint8_t* packed_out, void* scales_out,
                 float* tensor_scale, int tensor_scale_mode, rhtq_stream_t stream) {
  if (in_dtype != RHTQ_IN_BF16 && in_dtype != RHTQ_IN_F16 && in_dtype != RHTQ_IN_F32) return RHTQ_EINVAL;
  rhtq::KernelArgs a{};
  int st = shape_args(tokens, n, block, a);
  if (st == RHTQ_OK) st = check_quant_block(n, block, fmt, group, scale_dtype);
  if (st != RHTQ_OK) return st;
  if (fmt == RHTQ_FMT_NVFP4 && tensor_scale_mode != RHTQ_TENSOR_SCALE_DYNAMIC &&
      tensor_scale_mode != RHTQ_TENSOR_SCALE_GIVEN)
    return RHTQ_EINVAL;
  if (tokens == 0) return RHTQ_OK;
  if (!x || !packed_out || !scales_out) return RHTQ_EINVAL;
  if (fmt == RHTQ_FMT_NVFP4 && !tensor_scale) return RHTQ_EINVAL;
  if (!aligned(x, 16) || !aligned(packed_out, 16) || !aligned(scales_out, scale_align(scale_dtype)) ||
      !aligned(signs, 16))
    return RHTQ_EINVAL;
  if (fmt == RHTQ_FMT_NVFP4 && !aligned(tensor_scale, 4)) return RHTQ_EINVAL;

  a.x = x;
  a.signs = signs;
  a.group = group == 0 ? a.n : group;
  a.scale_dtype = scale_dtype;
  a.packed = packed_out;
  a.scales = scales_out;
  a.tensor_scale = tensor_scale;
  if (rhtq::getenv_test_fail_launch()) return RHTQ_EHIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  auto run = [&](int op) -> hipError_t {
    const hipError_t e = fast_for(in_dtype, op, a, s);
    if (e != hipErrorNotSupported) return e;
    return rhtq::launch_generic(op, in_dtype, a, s);
  };

  if (fmt == RHTQ_FMT_INT4) return from_hip(run(rhtq::OP_INT4));
  if (fmt == RHTQ_FMT_MXFP4) return from_hip(run(rhtq::OP_MXFP4));
  if (tensor_scale_mode == RHTQ_TENSOR_SCALE_DYNAMIC) {
    // the pre-pass leaves g itself in *tensor_scale (atomic max of per-workgroup g)
    hipError_t e = rhtq::launch_zero_word(tensor_scale, s);
    if (e == hipSuccess) e = run(rhtq::OP_AMAX);
    if (e != hipSuccess) return RHTQ_EHIP;
  }
  return from_hip(run(rhtq::OP_NVFP4));
}

int inverse_impl(const uint8_t* packed, const void* scales, const float* tensor_scale, int64_t tokens,
                 int32_t n, int32_t block, const int8_t* signs, int fmt, int32_t group, int scale_dtype,
                 float* x_out, rhtq_stream_t stream) {
  rhtq::KernelArgs a{};
  int st = shape_args(tokens, n, block, a);
  if (st == RHTQ_OK) st = check_quant_block(n, block, fmt, group, scale_dtype);
  if (st != RHTQ_OK) return st;
  if (tokens == 0) return RHTQ_OK;
  if (!packed || !scales || !x_out) return RHTQ_EINVAL;
  if (fmt == RHTQ_FMT_NVFP4 && !tensor_scale) return RHTQ_EINVAL;
  if (!aligned(packed, 4) || !aligned(x_out, 16) || !aligned(scales, scale_align(scale_dtype)) ||
      !aligned(signs, 16))
    return RHTQ_EINVAL;
  a.signs = signs;
  a.group = group == 0 ? a.n : group;
  a.scale_dtype = scale_dtype;
  a.y = x_out;
  a.in_packed = packed;
  a.in_scales = scales;
  a.in_tensor_scale = tensor_scale;
  a.inv_fmt = fmt;
  if (rhtq::getenv_test_fail_launch()) return RHTQ_EHIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (!rhtq::getenv_fast_disabled()) {
    const hipError_t e = rhtq::launch_inverse_fast(a, s);
    if (e != hipErrorNotSupported) return from_hip(e);
  }
  return from_hip(rhtq::launch_generic(rhtq::OP_INVERSE, RHTQ_IN_BF16, a, s));
}

}  // namespace

extern "C" {

int rhtq_abi_version(void) { return RHTQ_ABI_VERSION; }

const char* rhtq_status_str(int status) {
  switch (status) {
    case RHTQ_OK: return "ok";
    case RHTQ_EINVAL: return "invalid argument";
    case RHTQ_EUNSUPPORTED: return "unsupported width, format or group";
    case RHTQ_EHIP: return "HIP runtime error while enqueueing";
    default: return "unknown status";
  }
}

int rhtq_supported(int32_t n, int fmt, int32_t group) { return width_ok(n) && group_ok(n, fmt, group); }

int rhtq_rotate(const void* x, int in_dtype, int64_t tokens, int32_t n, const int8_t* signs,
                float* y_out, rhtq_stream_t stream) {
  return rotate_impl(x, in_dtype, tokens, n, n, signs, y_out, stream);
}

int rhtq_rotate_blocked(const void* x, int in_dtype, int64_t tokens, int32_t n, int32_t block,
                        const int8_t* signs, float* y_out, rhtq_stream_t stream) {
  return rotate_impl(x, in_dtype, tokens, n, block, signs, y_out, stream);
}

int rhtq_forward(const void* x, int in_dtype, int64_t tokens, int32_t n, const int8_t* signs, int fmt,
                 int32_t group, int scale_dtype, uint8_t* packed_out, void* scales_out,
                 float* tensor_scale, int tensor_scale_mode, rhtq_stream_t stream) {
  return forward_impl(x, in_dtype, tokens, n, n, signs, fmt, group, scale_dtype, packed_out, scales_out,
                      tensor_scale, tensor_scale_mode, stream);
}

int rhtq_forward_blocked(const void* x, int in_dtype, int64_t tokens, int32_t n, int32_t block,
                         const int8_t* signs, int fmt, int32_t group, int scale_dtype, uint8_t* packed_out,
                         void* scales_out, float* tensor_scale, int tensor_scale_mode,
                         rhtq_stream_t stream) {
  return forward_impl(x, in_dtype, tokens, n, block, signs, fmt, group, scale_dtype, packed_out, scales_out,
                      tensor_scale, tensor_scale_mode, stream);
}

int rhtq_inverse(const uint8_t* packed, const void* scales, const float* tensor_scale, int64_t tokens,
                 int32_t n, const int8_t* signs, int fmt, int32_t group, int scale_dtype, float* x_out,
                 rhtq_stream_t stream) {
  return inverse_impl(packed, scales, tensor_scale, tokens, n, n, signs, fmt, group, scale_dtype, x_out, stream);
}

int rhtq_inverse_blocked(const uint8_t* packed, const void* scales, const float* tensor_scale, int64_t tokens,
                         int32_t n, int32_t block, const int8_t* signs, int fmt, int32_t group, int scale_dtype,
                         float* x_out, rhtq_stream_t stream) {
  return inverse_impl(packed, scales, tensor_scale, tokens, n, block, signs, fmt, group, scale_dtype, x_out,
                      stream);
}

int rhtq_signs_from_seed(uint64_t seed, int32_t n, int8_t* host_out) {
  if (n < 0 || (n > 0 && !host_out)) return RHTQ_EINVAL;
  uint64_t state = seed;
  for (int32_t i = 0; i < n; ++i) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z = z ^ (z >> 31);
    host_out[i] = (z >> 63) ? -1 : 1;
  }
  return RHTQ_OK;
}

}  // extern "C"
