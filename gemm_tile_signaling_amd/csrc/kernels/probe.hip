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
// Design: the signaling GEMM's 256 x 128 tile in MFMAs alone.  512 threads
// (eight waves, two per SIMD) per workgroup; every lane reads 16 vectors of 16
// bytes from the buffer (indices wrap modulo the buffer's length): two sets
// of 4 A and 4 B fragments.  Each round runs, for each set in turn, the 4 x 4
// outer product of v_mfma_f32_16x16x32 that a wave's 64 x 64 sub-tile does per
// k-step (B fragment first, as in the GEMM), 32 MFMAs into 16 accumulators,
// so consecutive MFMAs share an A fragment and the operands change between
// k-steps as in the GEMM.  Each lane stores the sum of its accumulators, which
// keeps the work observable.
#include "../fo_internal.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

constexpr int kThreads = 512;
constexpr int kFrag = 4;  // A and B fragments per set: a 4 x 4 block grid of 16 x 16

template <typename T>
__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mma<__bf16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma<_Float16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(const u32x4 *ops, uint64_t n_vec, int32_t iters,
                                                             float *out) {
  const uint64_t lane_id = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 a[2][kFrag], b[2][kFrag];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int j = 0; j < kFrag; ++j) {
      a[u][j] = ops[(lane_id * 16 + u * 8 + j) % n_vec];
      b[u][j] = ops[(lane_id * 16 + u * 8 + kFrag + j) % n_vec];
    }
  f32x4 acc[kFrag][kFrag];
#pragma unroll
  for (int i = 0; i < kFrag; ++i)
#pragma unroll
    for (int j = 0; j < kFrag; ++j) acc[i][j] = f32x4{};
  for (int32_t it = 0; it < iters; ++it)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < kFrag; ++i)
#pragma unroll
        for (int j = 0; j < kFrag; ++j) acc[i][j] = mma<T>(b[u][j], a[u][i], acc[i][j]);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kFrag; ++i)
#pragma unroll
    for (int j = 0; j < kFrag; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) s += acc[i][j][r];
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
