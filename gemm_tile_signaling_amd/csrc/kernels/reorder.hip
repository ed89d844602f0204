// Pre- and post-communication reordering as standalone passes, and the
// post-communication reorder fused with the element-wise epilogue.
//
// Method: deep-dive page "FlashOverlap: 信号驱动计算通信重叠论文详解",
//   二、重排机制 › 解决方案: 映射表重排 -- after communication the inverse
//   mapping puts every tile back in place; 二 › 不同通信原语的重排模式
//   (Figure 6) for the three layouts.  The pre-communication direction is
//   normally fused into the GEMM epilogue; this pass exists for tests and
//   for layouts produced elsewhere.  五、CUTLASS 扩展实现 › Epilogue 集成 --
//   the element-wise operations after the GEMM (bias, ReLU, SiLU) run in the
//   post-communication reorder's pass, so the output is written once.
//
// Design: pure data movement, bound by HBM bandwidth.  One workgroup per
// (slot, band of up to 128 tile rows), over all slots or over the slots of a
// range of groups (a group's slots are consecutive); every row of a tile is a contiguous
// run of `cols` elements on both sides, so all accesses are 16-byte buffer
// loads and stores with 32-bit offsets (the plan keeps M*N at most 2^30).  The
// source and destination offset of each row are computed once into LDS;
// chunks outside the tile get an offset past the buffer's end, which the
// buffer bounds check turns into a zero load and a dropped store, so there
// are no branches; each thread issues all of its loads before its stores.
// Loads and stores are nontemporal: every byte is moved exactly once.
#include "../fo_internal.h"
#include "buffer.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
constexpr int kThreads = 256;
constexpr uint32_t kOutside = 0xFFFFFFF0u;  // byte offset past every buffer: zero load, dropped store
constexpr int kNT = 2;                       // buffer cache policy: nontemporal (each byte is moved once)

struct ReorderParams {
  const uint16_t *src;
  uint16_t *dst;
  const TileDesc *slots;
  Layout L;
  int64_t N;
  uint32_t bytes;  // 2 * M * N, the size of both buffers
  int32_t to_rowmajor;
  const uint16_t *bias;  // epilogue only: [problems][N], or NULL
  uint32_t bias_bytes;
  int32_t slot0;         // first slot of the launch: workgroup (x, y) moves slot slot0 + x
};

template <int RPB, int CPR>  // rows per block, 16-byte chunks per tile row
__global__ __launch_bounds__(kThreads) void reorder_kernel(ReorderParams p) {
  __shared__ uint32_t src_row[RPB], dst_row[RPB];  // byte offsets of each row's first element
  constexpr int kPer = RPB * CPR / kThreads;
  static_assert(RPB * CPR % kThreads == 0, "split");
  const int slot = p.slot0 + blockIdx.x;
  const int r0 = blockIdx.y * RPB;
  const TileDesc t = p.slots[slot];
  const int tid = threadIdx.x;
  if (tid < RPB && r0 + tid < t.rows) {
    const uint32_t reo = (uint32_t)row_offset(p.L, t, slot, r0 + tid) * 2u;
    const uint32_t rm = (uint32_t)((int64_t)(t.row0 + r0 + tid) * p.N + t.col0) * 2u;
    src_row[tid] = p.to_rowmajor ? reo : rm;
    dst_row[tid] = p.to_rowmajor ? rm : reo;
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.src, p.bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dst, p.bytes);
  u32x4 v[kPer];
  uint32_t dst_off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = tid + i * kThreads, r = q / CPR, c8 = q % CPR;
    const bool in = r0 + r < t.rows && c8 * 8 < t.cols;
    v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? src_row[r] + c8 * 16u : kOutside, 0, kNT);
    dst_off[i] = in ? dst_row[r] + c8 * 16u : kOutside;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) __builtin_amdgcn_raw_buffer_store_b128(v[i], rd, dst_off[i], 0, kNT);
}

typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  static __device__ __forceinline__ f32x8 widen(u32x4 v) { return __builtin_convertvector(__builtin_bit_cast(bf16x8, v), f32x8); }
  static __device__ __forceinline__ u32x4 narrow(f32x8 x) { return __builtin_bit_cast(u32x4, __builtin_convertvector(x, bf16x8)); }
};
template <>
struct Vec8<_Float16> {
  static __device__ __forceinline__ f32x8 widen(u32x4 v) { return __builtin_convertvector(__builtin_bit_cast(f16x8, v), f32x8); }
  static __device__ __forceinline__ u32x4 narrow(f32x8 x) { return __builtin_bit_cast(u32x4, __builtin_convertvector(x, f16x8)); }
};

// SiLU with the hardware exp2 and reciprocal instructions: both are within a
// few fp32 ulps, far below half an ulp of the 16-bit result, and they keep the
// pass bound by memory rather than by the vector ALU.  exp2 overflows to +inf
// for very negative x, whose reciprocal is 0: the result is -0, as x / inf.
template <int ACT>
__device__ __forceinline__ float act(float x) {
  if (ACT == FO_ACT_RELU) return x > 0.0f ? x : 0.0f;
  if (ACT == FO_ACT_SILU) return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
  return x;
}

// out[m, n] = round(act(float(recv[off(m, n)]) + float(bias[problem(m), n]))):
// the post-communication reorder with the element-wise epilogue.  Same grid
// and addressing as reorder_kernel in the row-major direction; a thread's
// 16-byte column chunk is the same for every row it moves (kThreads is a
// multiple of the chunks per row), so it loads its 8 bias values once.  One
// fp32 addition, the activation in fp32, one rounding to the element type.
template <typename T, int RPB, int CPR, int ACT, bool BIAS>
__global__ __launch_bounds__(kThreads) void post_ep_kernel(ReorderParams p) {
  __shared__ uint32_t src_row[RPB], dst_row[RPB];
  constexpr int kPer = RPB * CPR / kThreads;
  static_assert(RPB * CPR % kThreads == 0 && kThreads % CPR == 0, "split");
  const int slot = p.slot0 + blockIdx.x;
  const int r0 = blockIdx.y * RPB;
  const TileDesc t = p.slots[slot];
  const int tid = threadIdx.x;
  if (tid < RPB && r0 + tid < t.rows) {
    src_row[tid] = (uint32_t)row_offset(p.L, t, slot, r0 + tid) * 2u;
    dst_row[tid] = (uint32_t)((int64_t)(t.row0 + r0 + tid) * p.N + t.col0) * 2u;
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.src, p.bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dst, p.bytes);
  const int c8 = tid % CPR;
  f32x8 b = {};
  if (BIAS) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bias, p.bias_bytes);
    const uint32_t boff = c8 * 8 < t.cols ? (uint32_t)((int64_t)t.problem * p.N + t.col0 + c8 * 8) * 2u : kOutside;
    b = Vec8<T>::widen(__builtin_amdgcn_raw_buffer_load_b128(rb, boff, 0, 0));
  }
  u32x4 v[kPer];
  uint32_t dst_off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = (tid + i * kThreads) / CPR;
    const bool in = r0 + r < t.rows && c8 * 8 < t.cols;
    v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? src_row[r] + c8 * 16u : kOutside, 0, kNT);
    dst_off[i] = in ? dst_row[r] + c8 * 16u : kOutside;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    f32x8 x = Vec8<T>::widen(v[i]);
    if (BIAS) x = x + b;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = act<ACT>(x[e]);
    __builtin_amdgcn_raw_buffer_store_b128(Vec8<T>::narrow(x), rd, dst_off[i], 0, kNT);
  }
}

template <typename T, int ACT, bool BIAS>
void launch_post_ep_typed(const fo_plan *p, const ReorderParams &rp, hipStream_t s) {
  if (p->BN == 128)
    hipLaunchKernelGGL((post_ep_kernel<T, 128, 16, ACT, BIAS>), dim3(p->NT, (p->BM + 127) / 128), dim3(kThreads), 0,
                       s, rp);
  else
    hipLaunchKernelGGL((post_ep_kernel<T, 64, 8, ACT, BIAS>), dim3(p->NT, (p->BM + 63) / 64), dim3(kThreads), 0, s,
                       rp);
}

template <typename T>
void launch_post_ep_act(const fo_plan *p, const ReorderParams &rp, int act, hipStream_t s) {
  const bool bias = rp.bias != nullptr;
  switch (act) {
    case FO_ACT_RELU:
      bias ? launch_post_ep_typed<T, FO_ACT_RELU, true>(p, rp, s) : launch_post_ep_typed<T, FO_ACT_RELU, false>(p, rp, s);
      break;
    case FO_ACT_SILU:
      bias ? launch_post_ep_typed<T, FO_ACT_SILU, true>(p, rp, s) : launch_post_ep_typed<T, FO_ACT_SILU, false>(p, rp, s);
      break;
    default:
      bias ? launch_post_ep_typed<T, FO_ACT_NONE, true>(p, rp, s) : launch_post_ep_typed<T, FO_ACT_NONE, false>(p, rp, s);
  }
}

}  // namespace

int launch_post_ep(const fo_plan *p, const void *src, void *dst, const void *bias, int act, hipStream_t s) {
  if (p->NT == 0) return FO_OK;
  if (p->BN != 128 && p->BN != 64) return FO_ERR_UNSUPPORTED;
  ReorderParams rp{};
  rp.src = static_cast<const uint16_t *>(src);
  rp.dst = static_cast<uint16_t *>(dst);
  rp.slots = p->d_slots;
  rp.L = p->layout(true);
  rp.N = p->N;
  rp.bytes = (uint32_t)(2 * p->M * p->N);
  rp.to_rowmajor = 1;
  rp.bias = static_cast<const uint16_t *>(bias);
  rp.bias_bytes = (uint32_t)(2 * (int64_t)p->num_problems * p->N);
  if (p->dtype == FO_BF16)
    launch_post_ep_act<__bf16>(p, rp, act, s);
  else
    launch_post_ep_act<_Float16>(p, rp, act, s);
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

int launch_reorder(const fo_plan *p, const void *src, void *dst, bool to_rowmajor, int32_t slot_begin,
                   int32_t slot_end, hipStream_t s) {
  const int32_t nslots = slot_end - slot_begin;
  if (nslots <= 0) return FO_OK;
  ReorderParams rp{};
  rp.src = static_cast<const uint16_t *>(src);
  rp.dst = static_cast<uint16_t *>(dst);
  rp.slots = p->d_slots;
  rp.L = p->layout(true);
  rp.N = p->N;
  rp.bytes = (uint32_t)(2 * p->M * p->N);
  rp.to_rowmajor = to_rowmajor ? 1 : 0;
  rp.slot0 = slot_begin;
  if (p->BN == 128) {
    constexpr int RPB = 128;
    hipLaunchKernelGGL((reorder_kernel<RPB, 16>), dim3(nslots, (p->BM + RPB - 1) / RPB), dim3(kThreads), 0, s, rp);
  } else if (p->BN == 64) {
    constexpr int RPB = 64;
    hipLaunchKernelGGL((reorder_kernel<RPB, 8>), dim3(nslots, (p->BM + RPB - 1) / RPB), dim3(kThreads), 0, s, rp);
  } else {
    return FO_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

}  // namespace fo
