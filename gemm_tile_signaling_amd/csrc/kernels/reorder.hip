// Pre- and post-communication reordering as standalone passes.
//
// Method: deep-dive page "FlashOverlap: 信号驱动计算通信重叠论文详解",
//   二、重排机制 › 解决方案: 映射表重排 -- after communication the inverse
//   mapping puts every tile back in place; 二 › 不同通信原语的重排模式
//   (Figure 6) for the three layouts.  The pre-communication direction is
//   normally fused into the GEMM epilogue; this pass exists for tests and
//   for layouts produced elsewhere.
//
// Design: pure data movement, bound by HBM bandwidth.  One workgroup per
// (slot, band of up to 128 tile rows); every row of a tile is a contiguous
// run of `cols` elements on both sides, so all accesses are 16-byte vector
// loads and stores.  The destination/source offset of each row is computed
// once into LDS, then each thread issues all of its loads before its stores.
#include "../fo_internal.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
constexpr int kThreads = 256;

struct ReorderParams {
  const uint16_t *src;
  uint16_t *dst;
  const TileDesc *slots;
  Layout L;
  int64_t N;
  int32_t to_rowmajor;
};

template <int RPB, int CPR>  // rows per block, 16-byte chunks per tile row
__global__ __launch_bounds__(kThreads) void reorder_kernel(ReorderParams p) {
  __shared__ int64_t ro[RPB];
  constexpr int kPer = RPB * CPR / kThreads;
  static_assert(RPB * CPR % kThreads == 0, "split");
  const int slot = blockIdx.x;
  const int r0 = blockIdx.y * RPB;
  const TileDesc t = p.slots[slot];
  const int tid = threadIdx.x;
  if (tid < RPB && r0 + tid < t.rows) ro[tid] = row_offset(p.L, t, slot, r0 + tid);
  __syncthreads();
  u32x4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = tid + i * kThreads, r = q / CPR, c8 = q % CPR;
    if (r0 + r < t.rows && c8 * 8 < t.cols) {
      const int64_t rm = (int64_t)(t.row0 + r0 + r) * p.N + t.col0 + c8 * 8;
      const int64_t src = p.to_rowmajor ? ro[r] + c8 * 8 : rm;
      v[i] = *reinterpret_cast<const u32x4 *>(p.src + src);
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = tid + i * kThreads, r = q / CPR, c8 = q % CPR;
    if (r0 + r < t.rows && c8 * 8 < t.cols) {
      const int64_t rm = (int64_t)(t.row0 + r0 + r) * p.N + t.col0 + c8 * 8;
      const int64_t dst = p.to_rowmajor ? rm : ro[r] + c8 * 8;
      *reinterpret_cast<u32x4 *>(p.dst + dst) = v[i];
    }
  }
}

}  // namespace

int launch_reorder(const fo_plan *p, const void *src, void *dst, bool to_rowmajor, hipStream_t s) {
  if (p->NT == 0) return FO_OK;
  ReorderParams rp{};
  rp.src = static_cast<const uint16_t *>(src);
  rp.dst = static_cast<uint16_t *>(dst);
  rp.slots = p->d_slots;
  rp.L = p->layout(true);
  rp.N = p->N;
  rp.to_rowmajor = to_rowmajor ? 1 : 0;
  if (p->BN == 128) {
    constexpr int RPB = 128;
    hipLaunchKernelGGL((reorder_kernel<RPB, 16>), dim3(p->NT, (p->BM + RPB - 1) / RPB), dim3(kThreads), 0, s, rp);
  } else if (p->BN == 64) {
    constexpr int RPB = 64;
    hipLaunchKernelGGL((reorder_kernel<RPB, 8>), dim3(p->NT, (p->BM + RPB - 1) / RPB), dim3(kThreads), 0, s, rp);
  } else {
    return FO_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

}  // namespace fo
