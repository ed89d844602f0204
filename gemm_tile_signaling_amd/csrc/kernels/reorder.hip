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
// run of `cols` elements on both sides, so all accesses are 16-byte buffer
// loads and stores with 32-bit offsets (the plan keeps M*N below 2^31).  The
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
};

template <int RPB, int CPR>  // rows per block, 16-byte chunks per tile row
__global__ __launch_bounds__(kThreads) void reorder_kernel(ReorderParams p) {
  __shared__ uint32_t src_row[RPB], dst_row[RPB];  // byte offsets of each row's first element
  constexpr int kPer = RPB * CPR / kThreads;
  static_assert(RPB * CPR % kThreads == 0, "split");
  const int slot = blockIdx.x;
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

}  // namespace

int launch_reorder(const fo_plan *p, const void *src, void *dst, bool to_rowmajor, hipStream_t s) {
  if (p->NT == 0) return FO_OK;
  ReorderParams rp{};
  rp.src = static_cast<const uint16_t *>(src);
  rp.dst = static_cast<uint16_t *>(dst);
  rp.slots = p->d_slots;
  rp.L = p->layout(true);
  rp.N = p->N;
  rp.bytes = (uint32_t)(2 * p->M * p->N);
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
