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
// (slot, band of up to 256 tile rows), over all slots or over the slots of a
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

#include <algorithm>

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
  // Row-major side of the move: row m at m * N, or, with shard_rows > 0, at
  // shard_row(m) * N, the row's place in the gathered ReduceScatter shards.
  int32_t shard_rows;    // M / R (0: plain row-major)
  int32_t band_rows;     // BM / R
  int32_t BM;
  uint32_t bytes;  // 2 * M * N, the size of both buffers
  int32_t to_rowmajor;
  const uint16_t *bias;  // epilogue only: [problems][N], or NULL
  uint32_t bias_bytes;
  int32_t slot0;         // first slot of the launch: workgroup (x, y) moves slot slot0 + x
};

// Rank k of R owns the rows whose band inside their tile row is k (rows m
// with floor((m mod BM) / (BM/R)) == k), kept as a shard in increasing row
// order; the shards lie back to back.  Row m's place among them.  Problems
// start at multiples of BM, so m mod BM is the row inside its tile.
__host__ __device__ __forceinline__ int64_t shard_row(int64_t m, int32_t BM, int32_t band, int32_t shard_rows) {
  const int64_t r = m % BM;
  return (r / band) * shard_rows + (m / BM) * band + r % band;
}

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
    const int64_t m = t.row0 + r0 + tid;
    const int64_t row = p.shard_rows ? shard_row(m, p.BM, p.band_rows, p.shard_rows) : m;
    const uint32_t rm = (uint32_t)(row * p.N + t.col0) * 2u;
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
// pass bound by memory rather than by the vector ALU.  One path for every x:
// e = 2^64 e^-|x| (at most 2^64, and normal in fp32 down to |x| = 132, where
// the hardware exp2 would flush e^-|x| itself to zero), and the logistic of x
// is 2^64 / (2^64 + e) for x >= 0 and e / (2^64 + e) below, so results into
// the bf16 denormals keep their value; x = -inf gives NaN, as x / (1 + e^-x)
// does (-inf times a zero logistic).
template <int ACT>
__device__ __forceinline__ float act(float x) {
  constexpr float kLog2e = 1.4426950408889634f;
  if (ACT == FO_ACT_RELU) return x > 0.0f ? x : 0.0f;
  if (ACT == FO_ACT_SILU) {
    const float e = __builtin_amdgcn_exp2f(64.0f - __builtin_fabsf(x) * kLog2e);
    return x * ((x >= 0.0f ? 0x1p64f : e) * __builtin_amdgcn_rcpf(0x1p64f + e));
  }
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

// out row m = gathered row shard_row(m): the block-cyclic row exchange after
// the AllGather of the ReduceScatter shards, with the element-wise epilogue.
// Only M, BM and R are needed (no per-slot records).  Workgroup (x, y) moves
// rows [x*RB, x*RB + RB) and the 16-byte column chunks y*256 + tid, y*256 +
// tid + gridDim.y*256, ...; a thread keeps its RB loads in flight, then
// stores.  Every row of a problem shares the problem's bias row: the problem
// of a row is found among the problems' first rows (a wave-uniform search).
constexpr int kRowsPerBlock = 8;

struct ExchangeParams {
  const uint16_t *src;
  uint16_t *dst;
  const uint16_t *bias;
  const int32_t *problem_row0;  // num_problems + 1
  int32_t num_problems;
  int32_t M, BM, band, shard_rows;
  int32_t cpr;                  // 16-byte chunks per row (N / 8)
  uint32_t bytes, bias_bytes;
  int64_t N;
};

template <typename T, int ACT, bool BIAS>
__global__ __launch_bounds__(kThreads) void row_exchange_kernel(ExchangeParams p) {
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * kRowsPerBlock;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.src, p.bytes);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dst, p.bytes);
  for (int32_t c8 = blockIdx.y * kThreads + tid; c8 - tid < p.cpr; c8 += gridDim.y * kThreads) {
    const bool col_in = c8 < p.cpr;
    u32x4 v[kRowsPerBlock];
    uint32_t dst_off[kRowsPerBlock];
    int32_t prob[kRowsPerBlock];
#pragma unroll
    for (int i = 0; i < kRowsPerBlock; ++i) {
      const int64_t m = m0 + i;
      const bool in = col_in && m < p.M;
      const int64_t src_row = shard_row(m, p.BM, p.band, p.shard_rows);
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? (uint32_t)(src_row * p.N * 2 + (int64_t)c8 * 16) : kOutside, 0,
                                                   kNT);
      dst_off[i] = in ? (uint32_t)(m * p.N * 2 + (int64_t)c8 * 16) : kOutside;
      int32_t e = 0;  // problem of row m: problem_row0[e] <= m < problem_row0[e + 1]
      if (BIAS)
        while (e + 1 < p.num_problems && p.problem_row0[e + 1] <= m) ++e;
      prob[i] = e;
    }
#pragma unroll
    for (int i = 0; i < kRowsPerBlock; ++i) {
      f32x8 x = Vec8<T>::widen(v[i]);
      if (BIAS) {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bias, p.bias_bytes);
        const uint32_t boff = col_in ? (uint32_t)((int64_t)prob[i] * p.N * 2 + (int64_t)c8 * 16) : kOutside;
        x = x + Vec8<T>::widen(__builtin_amdgcn_raw_buffer_load_b128(rb, boff, 0, 0));
      }
      if (ACT != FO_ACT_NONE) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = act<ACT>(x[e]);
      }
      // without bias or activation the value is passed through untouched (no rounding step)
      const u32x4 o = (BIAS || ACT != FO_ACT_NONE) ? Vec8<T>::narrow(x) : v[i];
      __builtin_amdgcn_raw_buffer_store_b128(o, rd, dst_off[i], 0, kNT);
    }
  }
}

template <typename T, int ACT, bool BIAS>
void launch_post_ep_typed(const fo_plan *p, const ReorderParams &rp, hipStream_t s) {
  if (p->BN == 256)
    hipLaunchKernelGGL((post_ep_kernel<T, 64, 32, ACT, BIAS>), dim3(p->NT, (p->BM + 63) / 64), dim3(kThreads), 0, s,
                       rp);
  else if (p->BN == 128)
    hipLaunchKernelGGL((post_ep_kernel<T, 256, 16, ACT, BIAS>), dim3(p->NT, (p->BM + 255) / 256), dim3(kThreads), 0,
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

int launch_reorder_params(const fo_plan *p, const ReorderParams &rp, int32_t nslots, hipStream_t s) {
  if (p->BN == 256) {
    constexpr int RPB = 64;
    hipLaunchKernelGGL((reorder_kernel<RPB, 32>), dim3(nslots, (p->BM + RPB - 1) / RPB), dim3(kThreads), 0, s, rp);
  } else if (p->BN == 128) {
    // a whole tile of up to 256 rows per workgroup, 16 chunks in flight per
    // thread: 5% faster than bands of 128 rows on 32 MiB (82 registers, which
    // fit beside the 256 x 128 GEMM's two 192-register waves)
    constexpr int RPB = 256;
    hipLaunchKernelGGL((reorder_kernel<RPB, 16>), dim3(nslots, (p->BM + RPB - 1) / RPB), dim3(kThreads), 0, s, rp);
  } else if (p->BN == 64) {
    constexpr int RPB = 64;
    hipLaunchKernelGGL((reorder_kernel<RPB, 8>), dim3(nslots, (p->BM + RPB - 1) / RPB), dim3(kThreads), 0, s, rp);
  } else {
    return FO_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

template <typename T, int ACT>
void launch_exchange_act(const ExchangeParams &ep, dim3 grid, hipStream_t s) {
  if (ep.bias)
    hipLaunchKernelGGL((row_exchange_kernel<T, ACT, true>), grid, dim3(kThreads), 0, s, ep);
  else
    hipLaunchKernelGGL((row_exchange_kernel<T, ACT, false>), grid, dim3(kThreads), 0, s, ep);
}

template <typename T>
void launch_exchange_typed(const ExchangeParams &ep, int act, dim3 grid, hipStream_t s) {
  switch (act) {
    case FO_ACT_RELU: launch_exchange_act<T, FO_ACT_RELU>(ep, grid, s); break;
    case FO_ACT_SILU: launch_exchange_act<T, FO_ACT_SILU>(ep, grid, s); break;
    default: launch_exchange_act<T, FO_ACT_NONE>(ep, grid, s);
  }
}

}  // namespace

int launch_post_ep(const fo_plan *p, const void *src, void *dst, const void *bias, int act, hipStream_t s) {
  if (p->NT == 0) return FO_OK;
  if (p->BN != 256 && p->BN != 128 && p->BN != 64) return FO_ERR_UNSUPPORTED;
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

int launch_row_exchange(const fo_plan *p, const void *gathered, void *out, const void *bias, int act,
                        hipStream_t s) {
  if (p->M == 0) return FO_OK;
  ExchangeParams ep{};
  ep.src = static_cast<const uint16_t *>(gathered);
  ep.dst = static_cast<uint16_t *>(out);
  ep.bias = static_cast<const uint16_t *>(bias);
  ep.problem_row0 = p->d_problem_row0;
  ep.num_problems = p->num_problems;
  ep.M = (int32_t)p->M;
  ep.BM = p->BM;
  ep.band = p->band_rows;
  ep.shard_rows = (int32_t)(p->M / p->ranks);
  ep.cpr = (int32_t)(p->N / 8);
  ep.bytes = (uint32_t)(2 * p->M * p->N);
  ep.bias_bytes = (uint32_t)(2 * (int64_t)p->num_problems * p->N);
  ep.N = p->N;
  const int64_t col_blocks = (ep.cpr + kThreads - 1) / kThreads;
  const dim3 grid((uint32_t)((p->M + kRowsPerBlock - 1) / kRowsPerBlock), (uint32_t)std::min<int64_t>(col_blocks, 1024));
  if (p->dtype == FO_BF16)
    launch_exchange_typed<__bf16>(ep, act, grid, s);
  else
    launch_exchange_typed<_Float16>(ep, act, grid, s);
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

int launch_shards(const fo_plan *p, const void *src, void *gathered, hipStream_t s) {
  if (p->NT == 0) return FO_OK;
  ReorderParams rp{};
  rp.src = static_cast<const uint16_t *>(src);
  rp.dst = static_cast<uint16_t *>(gathered);
  rp.slots = p->d_slots;
  rp.L = p->layout(true);
  rp.N = p->N;
  rp.bytes = (uint32_t)(2 * p->M * p->N);
  rp.to_rowmajor = 1;
  rp.shard_rows = (int32_t)(p->M / p->ranks);
  rp.band_rows = p->band_rows;
  rp.BM = p->BM;
  rp.slot0 = 0;
  return launch_reorder_params(p, rp, p->NT, s);
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
  return launch_reorder_params(p, rp, nslots, s);
}

}  // namespace fo
