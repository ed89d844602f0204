// Signaling GEMM for gfx950: C = A . B^T, bf16/fp16 in, fp32 accumulate.
//
// Method: deep-dive page "FlashOverlap: 信号驱动计算通信重叠论文详解",
//   五、CUTLASS 扩展实现 › 扩展主循环 / Epilogue 集成 -- the main loop is an
//   ordinary GEMM; the epilogue stores each finished tile through the mapping
//   table and updates the counting table; 一、信号机制 › 实现方法: 组级 Tile
//   计数 -- the group whose entry reaches |G_j| is signalled.
//
// Design (MI355X, not the pages' CUTLASS design):
//   * persistent grid of exactly W workgroups (W = wave size); workgroup g
//     runs dispatch indices pos(g), pos(g) + W, ... so wave w is every
//     workgroup's w-th tile.  pos() packs each XCD's workgroups (hardware
//     places workgroup g on XCD g % 8) onto a contiguous run of positions of
//     the wave, so the tiles sharing an XCD's L2 are neighbours in the
//     swizzled order.  This only permutes workgroups inside a wave.
//   * 256 threads = 4 waves in a 2 x 2 grid; each wave owns a (BM/2) x (BN/2)
//     sub-tile made of 32 x 32 blocks computed with v_mfma_f32_32x32x16.
//     A and B fragments are passed to the MFMA swapped (B as the first
//     operand) so that every lane ends up with 4 consecutive columns of one
//     output row, which the epilogue writes as 8-byte pieces.
//   * BK = 64; A and B tiles are staged through LDS in two buffers: the
//     global loads of slice k+1 are in flight while slice k is multiplied.
//     LDS rows are 128 bytes (64 K-elements); 16-byte chunk c of row r is
//     stored at chunk c ^ (r & 7), so the eight lanes of a ds_read_b128
//     phase that read the same K-chunk of eight consecutive rows hit eight
//     different bank groups.
//   * Global loads are buffer loads against a per-tile resource whose size
//     ends at the tile's last valid row, so rows past an edge read zeros and
//     never touch memory outside the problem.
//   * Epilogue: accumulators -> 16-bit -> LDS staging tile; every valid row's
//     destination offset (row-major, banded or subtoken layout) is computed
//     once into LDS; then 16-byte coalesced stores.  With signaling on, each
//     wave waits for its stores to complete, the workgroup meets at a
//     barrier, and one lane releases the tile to device scope and increments
//     cnt[group]; the lane that brings it to epoch * |G_group| stores
//     flag[group] = epoch with release semantics.
#include "../fo_internal.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int kRowBytes = BK * 2;               // one staged row of A or B
constexpr uint32_t kRsrcWord3 = 0x00020000u;    // raw buffer, 32-bit data format
constexpr int kVmcntZero = 0x0F70;              // s_waitcnt vmcnt(0), other counters unconstrained

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
__device__ __forceinline__ u32x2 pack4(f32x4 v);
template <>
__device__ __forceinline__ u32x2 pack4<__bf16>(f32x4 v) {
  return __builtin_bit_cast(u32x2, __builtin_convertvector(v, bf16x4));
}
template <>
__device__ __forceinline__ u32x2 pack4<_Float16>(f32x4 v) {
  return __builtin_bit_cast(u32x2, __builtin_convertvector(v, f16x4));
}

struct GemmParams {
  const uint16_t *A;
  const uint16_t *B;
  uint16_t *C;
  const TileDesc *slots;
  int32_t NT, W, K, remap;
  int64_t b_stride;        // elements between consecutive problems' B
  Layout L;
  uint32_t *cnt;           // NULL: no signaling
  uint32_t *flag;
  const int32_t *thr;      // |G_j|
  uint64_t *trace;
  uint32_t epoch;
  int32_t P;
};

template <int BM, int BN>
struct Cfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_PER_T = BM * 8 / kThreads;  // 16-byte chunks per thread per stage
  static constexpr int B_PER_T = BN * 8 / kThreads;
  static constexpr int STAGE = (BM + BN) * kRowBytes;
  static constexpr int OUT_PITCH = BN * 2 + 16;      // bytes per staged output row
  static constexpr int OUT_BYTES = BM * OUT_PITCH;
  static constexpr int ROWOFF = OUT_BYTES;           // int64 per row after the staging tile
  static constexpr int LDS = (2 * STAGE > OUT_BYTES + BM * 8) ? 2 * STAGE : OUT_BYTES + BM * 8;
  static_assert(BM * 8 % kThreads == 0 && BN * 8 % kThreads == 0, "chunk split");
  static_assert(FM >= 1 && FN >= 1, "wave tile");
};

template <typename T, int BM, int BN>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmParams p) {
  using C = Cfg<BM, BN>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = blockIdx.x;
  const int pos = p.remap ? (g & 7) * (p.W >> 3) + (g >> 3) : g;
  const int nk = p.K / BK;
  const uint32_t row_bytes = (uint32_t)p.K * 2u;

  // global -> LDS copy coordinates.  Chunk i of a thread is row tid/8 + 32 i,
  // 16-byte column tid % 8; the row's swizzle term (row & 7) does not depend
  // on i, so one base offset per operand plus compile-time strides suffices.
  const uint32_t g_base = (uint32_t)(tid >> 3) * row_bytes + (uint32_t)(tid & 7) * 16u;
  const uint32_t g_step = 32u * row_bytes;
  const uint32_t s_base = (uint32_t)((tid >> 3) * kRowBytes + (((tid & 7) ^ ((tid >> 3) & 7)) << 4));
  constexpr uint32_t s_step = 32u * kRowBytes;
  constexpr uint32_t s_bofs = BM * kRowBytes;      // B rows follow A rows in a stage
  // MFMA fragment reads: row (lane % 32) of each 32-row block, K-chunk ks*2 + lane/32
  const int frag_row = lane & 31, frag_half = lane >> 5, swz = lane & 7;
  const uint32_t a_frag = (uint32_t)((wm * C::WM + frag_row) * kRowBytes);
  const uint32_t b_frag = (uint32_t)(s_bofs + (wn * C::WN + frag_row) * kRowBytes);

  int64_t *rowoff = reinterpret_cast<int64_t *>(smem + C::ROWOFF);

  for (int b = pos; b < p.NT; b += p.W) {
    const TileDesc t = p.slots[b];
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.A + (int64_t)t.row0 * p.K), (short)0, (int)(t.rows * row_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.B + (int64_t)t.problem * p.b_stride + (int64_t)t.col0 * p.K), (short)0,
        (int)(t.cols * row_bytes), kRsrcWord3);

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

    u32x4 va[C::A_PER_T], vb[C::B_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) va[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, g_base + i * g_step, 0, 0);
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, g_base + i * g_step, 0, 0);
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) *reinterpret_cast<u32x4 *>(smem + s_base + i * s_step) = va[i];
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) *reinterpret_cast<u32x4 *>(smem + s_bofs + s_base + i * s_step) = vb[i];
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = (kt & 1) * C::STAGE;
      const bool more = kt + 1 < nk;
      if (more) {
        const int soff = (kt + 1) * kRowBytes;
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i)
          va[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, g_base + i * g_step, soff, 0);
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i)
          vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, g_base + i * g_step, soff, 0);
      }
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const uint32_t chunk = (uint32_t)(((ks * 2 + frag_half) ^ swz) << 4);
        u32x4 af[C::FM], bfr[C::FN];
#pragma unroll
        for (int f = 0; f < C::FM; ++f)
          af[f] = *reinterpret_cast<const u32x4 *>(smem + cur + a_frag + f * 32 * kRowBytes + chunk);
#pragma unroll
        for (int f = 0; f < C::FN; ++f)
          bfr[f] = *reinterpret_cast<const u32x4 *>(smem + cur + b_frag + f * 32 * kRowBytes + chunk);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) acc[i][j] = mma<T>(bfr[j], af[i], acc[i][j]);
      }
      if (more) {
        const int nxt = ((kt + 1) & 1) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i) *reinterpret_cast<u32x4 *>(smem + nxt + s_base + i * s_step) = va[i];
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i)
          *reinterpret_cast<u32x4 *>(smem + nxt + s_bofs + s_base + i * s_step) = vb[i];
      }
      __syncthreads();
    }

    // ---- epilogue: destination of every valid row, then the 16-bit tile through LDS
    if (tid < BM) rowoff[tid] = tid < t.rows ? row_offset(p.L, t, b, tid) : 0;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int r = wm * C::WM + i * 32 + frag_row;
          const int c = wn * C::WN + j * 32 + g4 * 8 + frag_half * 4;
          const f32x4 v = {acc[i][j][g4 * 4 + 0], acc[i][j][g4 * 4 + 1], acc[i][j][g4 * 4 + 2], acc[i][j][g4 * 4 + 3]};
          *reinterpret_cast<u32x2 *>(smem + r * C::OUT_PITCH + c * 2) = pack4<T>(v);
        }
    __syncthreads();
    constexpr int CPR = BN / 8;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < BM * CPR / kThreads; ++i) {
      const int q = tid + i * kThreads, r = q / CPR, c8 = q % CPR;
      if (r < t.rows && c8 * 8 < t.cols) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + r * C::OUT_PITCH + c8 * 16);
        *reinterpret_cast<u32x4 *>(p.C + rowoff[r] + c8 * 8) = v;
      }
    }

    // ---- signal: counting table, then the group's flag
    if (p.cnt) {
      // Each wave waits until its own tile stores are complete; after the
      // barrier one lane releases the whole workgroup's stores to device scope
      // (a single L2 write-back per tile) before it counts the tile.
      __builtin_amdgcn_s_waitcnt(kVmcntZero);
      __syncthreads();
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t old = __hip_atomic_fetch_add(&p.cnt[t.group], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool fire = old + 1u == p.epoch * (uint32_t)p.thr[t.group];
        if (fire) __hip_atomic_store(&p.flag[t.group], p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        if (p.trace) {
          p.trace[2 * (int64_t)b] = wall_clock64();
          p.trace[2 * (int64_t)b + 1] = ((uint64_t)(uint32_t)g << 32) | old;
          if (fire) __hip_atomic_fetch_add(&p.trace[2 * (int64_t)p.NT + t.group], (uint64_t)1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();  // the next tile's first stage overwrites the staging area
  }
}

template <typename T, int BM, int BN>
int launch_typed(const GemmParams &gp, hipStream_t s) {
  using C = Cfg<BM, BN>;
  static bool configured = false;  // per process; the attribute is per kernel and device-independent
  if (!configured) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_kernel<T, BM, BN>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS) != hipSuccess)
      return FO_ERR_HIP;
    configured = true;
  }
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN>), dim3(gp.W), dim3(kThreads), C::LDS, s, gp);
  return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
}

template <typename T>
int launch_tile(const fo_plan *p, const GemmParams &gp, hipStream_t s) {
  if (p->BM == 256 && p->BN == 128) return launch_typed<T, 256, 128>(gp, s);
  if (p->BM == 128 && p->BN == 128) return launch_typed<T, 128, 128>(gp, s);
  if (p->BM == 64 && p->BN == 64) return launch_typed<T, 64, 64>(gp, s);
  return FO_ERR_UNSUPPORTED;
}

}  // namespace

int launch_gemm(const fo_plan *p, const void *A, const void *B, void *Cout, bool rowmajor, uint32_t *sig,
                uint32_t epoch, uint64_t *trace, hipStream_t s) {
  if (p->NT == 0) return FO_OK;
  GemmParams gp{};
  gp.A = static_cast<const uint16_t *>(A);
  gp.B = static_cast<const uint16_t *>(B);
  gp.C = static_cast<uint16_t *>(Cout);
  gp.slots = p->d_slots;
  gp.NT = p->NT;
  gp.W = p->W;
  gp.K = (int32_t)p->K;
  gp.remap = (p->W % 8 == 0) ? 1 : 0;
  gp.b_stride = p->N * p->K;
  gp.L = p->layout(true);
  if (rowmajor) gp.L.mode = kRowMajor;
  gp.cnt = sig;
  gp.flag = sig ? sig + p->P : nullptr;
  gp.thr = p->d_group_tiles;
  gp.trace = sig ? trace : nullptr;
  gp.epoch = epoch;
  gp.P = p->P;
  return p->dtype == FO_BF16 ? launch_tile<__bf16>(p, gp, s) : launch_tile<_Float16>(p, gp, s);
}

}  // namespace fo
