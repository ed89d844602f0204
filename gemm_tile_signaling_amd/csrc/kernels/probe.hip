// Matrix-pipe rate on given operand values: a measurement aid for the
// signaling GEMM's roofline, not a step of the method.
//
// The GEMM's MFMA peak is a nominal figure (every CU issuing v_mfma at the
// top clock).  How close a kernel can come depends on the clock the part
// keeps under load, and under the power cap that clock depends on what the
// matrix pipe multiplies: random 16-bit mantissas toggle far more of its
// multipliers than constant or sparse values.  This kernel issues nothing but
// MFMAs on operand registers taken from a caller's buffer (for example the
// GEMM's own A), so its rate is the ceiling that operand values and the power
// cap leave for any kernel on the same data, without loads, LDS or epilogue.
//
// Design: 256 threads (four waves, one per SIMD) per workgroup.  Every lane
// reads 2 * kChains 16-byte vectors from the buffer (indices wrap modulo the
// buffer's length), then runs `iters` rounds of kChains independent
// v_mfma_f32_32x32x16 (enough independent accumulators to cover the
// instruction's latency), each chain with its own A and B operands, so
// consecutive MFMAs see different values as in a GEMM.  Each lane stores the
// sum of its accumulators, which keeps the work observable.
#include "../fo_internal.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

constexpr int kThreads = 256;
constexpr int kChains = 8;

template <typename T>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mma<__bf16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mma<_Float16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(const u32x4 *ops, uint64_t n_vec, int32_t iters,
                                                             float *out) {
  const uint64_t lane_id = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 a[kChains], b[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    a[j] = ops[(lane_id * 2 * kChains + j) % n_vec];
    b[j] = ops[(lane_id * 2 * kChains + kChains + j) % n_vec];
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x16{};
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = mma<T>(a[j], b[j], acc[j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[lane_id] = s;
}

}  // namespace

int launch_mfma_rate(int dtype, const void *ops, int64_t ops_bytes, int32_t workgroups, int32_t iters, float *out,
                     hipStream_t s) {
  const u32x4 *v = static_cast<const u32x4 *>(ops);
  const uint64_t n_vec = (uint64_t)ops_bytes / 16u;
  if (dtype == FO_BF16)
    hipLaunchKernelGGL(mfma_rate_kernel<__bf16>, dim3(workgroups), dim3(kThreads), 0, s, v, n_vec, iters, out);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<_Float16>, dim3(workgroups), dim3(kThreads), 0, s, v, n_vec, iters, out);
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

}  // namespace fo
