// Consumer: waits on the device for each wave group's signal, then reduces the
// group's contiguous span with a second buffer -- the one-GPU stand-in for the
// group's collective call.
//
// Method: deep-dive page "FlashOverlap: 信号驱动计算通信重叠论文详解",
//   五、CUTLASS 扩展实现 › 专用监控内核 -- progress is tracked through atomic
//   counters and communication runs on its own stream, notified by the
//   signals; 核心设计 › 通信侧 and 二 › (1) AllReduce (code box) -- the
//   contiguous span is handed to one collective call.
//
// Design: a persistent grid.  Every workgroup walks the groups in firing
// order; for each group one lane polls flag[g] (agent-scope loads, s_sleep
// back-off, bounded by the device wall clock), the workgroup meets at a
// barrier, and then all workgroups stream the group's span with 16-byte
// buffer loads: recv = round(float(send) + float(peer)).  The span is the
// concatenation of the group's work units (one per collective call in a
// multi-GPU consumer: the whole span, R rank segments or D destination
// buckets); the stand-in's reduction is the same on each, so it streams the
// span in one pass rather than paying a pass per unit.  The span is read
// with device-coherent loads (the cache policy that agent-scope atomic loads
// use), so data the producer published at device scope (written through its
// L2 and complete before the tile was counted) is read from the point of
// coherence and no workgroup has to invalidate its L2 (a full-L2
// invalidation per workgroup per group would evict the GEMM's operands and,
// with many workgroups, dominate the kernel).  The loads are nontemporal:
// each byte is read once, and streaming it past the caches roughly doubles
// the bandwidth a kernel of this shape reaches.  The stores of recv keep the
// default cache policy: the post-reorder reads recv right after this kernel,
// and writing it through the caches rather than streaming it to memory made
// the overlapped pass 2-4% shorter (the GEMM beside it 1-3% faster) with the
// kernel alone no slower.  Each span gets its own buffer
// resources, so the tail needs no branches: loads past the end read zeros and
// stores past the end are dropped.  The kernel holds no LDS beyond one word
// and few registers, so it can stay resident next to the GEMM's workgroups.
//
// The same kernel also runs as the second half of the gated consumer: a
// stream wait for the group's flag (hipStreamWaitValue32) is enqueued ahead
// of it, and it runs over that one group with a grid sized to the span; its
// single check of the flag then passes at once.
//
// Epoch stamps (optional, a plan flag): after a group's wait every workgroup
// reads its share of the group's per-slot stamps with the same device-coherent
// loads it uses for the span; a stamp other than the current epoch means the
// signal was seen before the tile it covers, and FO_ERR_STALE goes to the
// status word.
#include "../fo_internal.h"
#include "buffer.h"

#include <algorithm>

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;            // 16-byte chunks in flight per thread (4 was 5% slower gated)
// Beside a 256 x 256 GEMM workgroup (two 232-register waves per SIMD) a SIMD
// has 48 registers left: two chunks in flight per thread keep the consumer
// under that (43 registers against 89), so it can run beside the GEMM.
constexpr int kUnrollSlim = 2;
constexpr int kNT = 2;              // buffer cache policy: nontemporal (each byte is streamed once)
constexpr int kCoherent = 16;       // buffer cache policy: device-coherent load

struct ConsumeParams {
  const uint16_t *send;
  const uint16_t *peer;
  uint16_t *recv;
  const uint32_t *flag;
  const int64_t *unit_off;
  const int32_t *group_unit;
  const int32_t *group_first;  // first slot of each group (P + 1)
  const uint32_t *stamps;      // NULL, or one epoch stamp per slot
  int32_t *status;
  uint64_t *trace;         // NULL or [P]: wall clock when workgroup 0's wait for a group ended
  uint64_t timeout_ticks;
  uint32_t epoch;
  int32_t g_begin, g_end;
};

template <typename T>
__device__ __forceinline__ u32x4 add8(u32x4 a, u32x4 b);
template <>
__device__ __forceinline__ u32x4 add8<__bf16>(u32x4 a, u32x4 b) {
  const f32x8 x = __builtin_convertvector(__builtin_bit_cast(bf16x8, a), f32x8);
  const f32x8 y = __builtin_convertvector(__builtin_bit_cast(bf16x8, b), f32x8);
  return __builtin_bit_cast(u32x4, __builtin_convertvector(x + y, bf16x8));
}
template <>
__device__ __forceinline__ u32x4 add8<_Float16>(u32x4 a, u32x4 b) {
  const f32x8 x = __builtin_convertvector(__builtin_bit_cast(f16x8, a), f32x8);
  const f32x8 y = __builtin_convertvector(__builtin_bit_cast(f16x8, b), f32x8);
  return __builtin_bit_cast(u32x4, __builtin_convertvector(x + y, f16x8));
}

// flag values only grow, one step per launch; compare as a signed distance
__device__ __forceinline__ bool reached(uint32_t v, uint32_t epoch) { return (int32_t)(v - epoch) >= 0; }

__device__ __forceinline__ void record_status(int32_t *status, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(status, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// GATED: launched behind a stream wait for its one group (a grid sized to the
// span); the same code as the persistent form, instantiated apart so that
// kernel traces tell the two launch forms apart.
template <typename T, int UNROLL, bool GATED>
__global__ __launch_bounds__(kThreads) void consume_kernel(ConsumeParams p) {
  __shared__ int s_go;
  const int tid = threadIdx.x;
  const uint32_t stride = gridDim.x * kThreads;
  for (int g = p.g_begin; g < p.g_end; ++g) {
    if (tid == 0) {
      int go = 1;
      if (!reached(__hip_atomic_load(&p.flag[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), p.epoch)) {
        const uint64_t t0 = wall_clock64();
        for (;;) {
          __builtin_amdgcn_s_sleep(2);
          if (reached(__hip_atomic_load(&p.flag[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), p.epoch)) break;
          if (__hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
            go = 0;  // another workgroup gave up
            break;
          }
          if (wall_clock64() - t0 > p.timeout_ticks) {
            record_status(p.status, FO_ERR_TIMEOUT);
            go = 0;
            break;
          }
        }
      }
      s_go = go;
      if (go && p.trace && blockIdx.x == 0) p.trace[g] = wall_clock64();
    }
    __syncthreads();
    const int go = s_go;
    __syncthreads();  // s_go is rewritten for the next group
    if (!go) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no span load is hoisted above the wait

    if (p.stamps) {  // every tile of the group carries this epoch's stamp
      const int32_t s0 = p.group_first[g], s1 = p.group_first[g + 1];
      const __amdgpu_buffer_rsrc_t rt = make_rsrc(p.stamps + s0, (uint32_t)(s1 - s0) * 4u);
      for (int32_t i = blockIdx.x * kThreads + tid; i < s1 - s0; i += stride)
        if (__builtin_amdgcn_raw_buffer_load_b32(rt, (uint32_t)i * 4u, 0, kCoherent | kNT) != p.epoch)
          record_status(p.status, FO_ERR_STALE);
    }

    // The group's units tile its span back to back, and every unit gets the
    // same elementwise reduction, so the span is streamed as one range.
    const int64_t lo = p.unit_off[p.group_unit[g]], hi = p.unit_off[p.group_unit[g + 1]];  // multiples of 8
    const uint32_t bytes = (uint32_t)((hi - lo) * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.send + lo, bytes);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.peer + lo, bytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(p.recv + lo, bytes);
    const uint32_t n = bytes >> 4;  // 16-byte chunks in the span
    for (uint32_t c0 = blockIdx.x * kThreads + tid; c0 < n; c0 += UNROLL * stride) {
      u32x4 a[UNROLL], b[UNROLL];
#pragma unroll
      for (int i = 0; i < UNROLL; ++i) {
        const uint32_t off = (c0 + i * stride) * 16u;
        a[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCoherent | kNT);
        b[i] = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kNT);
      }
#pragma unroll
      for (int i = 0; i < UNROLL; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(add8<T>(a[i], b[i]), rr, (c0 + i * stride) * 16u, 0, 0);
    }
  }
}

ConsumeParams params(const fo_plan *p, const void *send, const void *peer, void *recv, const uint32_t *sig,
                     uint32_t epoch, int32_t g_begin, int32_t g_end, int32_t *status, uint64_t timeout_ticks,
                     uint64_t *trace) {
  ConsumeParams cp{};
  cp.send = static_cast<const uint16_t *>(send);
  cp.peer = static_cast<const uint16_t *>(peer);
  cp.recv = static_cast<uint16_t *>(recv);
  cp.flag = sig + p->flag_offset();
  cp.unit_off = p->d_unit_off;
  cp.group_unit = p->d_group_unit;
  cp.group_first = p->d_group_first;
  cp.stamps = p->stamps() ? sig + p->stamp_offset() : nullptr;
  cp.status = status;
  cp.trace = trace;
  cp.timeout_ticks = timeout_ticks;
  cp.epoch = epoch;
  cp.g_begin = g_begin;
  cp.g_end = g_end;
  return cp;
}

// The consumer's waves run beside the GEMM's on the same SIMDs: with a 256 x
// 256 GEMM tile only the slim form fits.
bool slim(const fo_plan *p) { return p->BM == 256 && p->BN == 256; }

template <bool GATED>
void launch_form(const fo_plan *p, const ConsumeParams &cp, int32_t grid, hipStream_t s) {
  const bool bf = p->dtype == FO_BF16;
  if (slim(p)) {
    if (bf)
      hipLaunchKernelGGL((consume_kernel<__bf16, kUnrollSlim, GATED>), dim3(grid), dim3(kThreads), 0, s, cp);
    else
      hipLaunchKernelGGL((consume_kernel<_Float16, kUnrollSlim, GATED>), dim3(grid), dim3(kThreads), 0, s, cp);
  } else {
    if (bf)
      hipLaunchKernelGGL((consume_kernel<__bf16, kUnroll, GATED>), dim3(grid), dim3(kThreads), 0, s, cp);
    else
      hipLaunchKernelGGL((consume_kernel<_Float16, kUnroll, GATED>), dim3(grid), dim3(kThreads), 0, s, cp);
  }
}

}  // namespace

int launch_consume(const fo_plan *p, const void *send, const void *peer, void *recv, const uint32_t *sig,
                   uint32_t epoch, int32_t g_begin, int32_t g_end, int32_t *status, uint64_t timeout_ticks,
                   int32_t grid, uint64_t *trace, hipStream_t s) {
  if (g_begin >= g_end) return FO_OK;
  const ConsumeParams cp = params(p, send, peer, recv, sig, epoch, g_begin, g_end, status, timeout_ticks, trace);
  launch_form<false>(p, cp, grid, s);
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

int launch_consume_ready(const fo_plan *p, const void *send, const void *peer, void *recv, const uint32_t *sig,
                         uint32_t epoch, int32_t g, int32_t *status, uint64_t *trace, hipStream_t s) {
  // enqueued behind a stream wait for the flag: the kernel's own wait passes at once
  const ConsumeParams cp = params(p, send, peer, recv, sig, epoch, g, g + 1, status, 2000000ull * p->ticks_per_us,
                                  trace);
  const int64_t chunks = (p->unit_off[p->group_unit[g + 1]] - p->unit_off[p->group_unit[g]]) / 8;
  const int64_t per_wg = (int64_t)kThreads * (slim(p) ? kUnrollSlim : kUnroll);
  const int32_t grid = (int32_t)std::min<int64_t>(std::max<int64_t>((chunks + per_wg - 1) / per_wg, 1), 16384);
  launch_form<true>(p, cp, grid, s);
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

}  // namespace fo
