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
//     deals consecutive workgroups round-robin over the 8 XCDs, so the
//     workgroups with one value of g % 8 share an XCD) onto a contiguous run
//     of positions of the wave, so the tiles sharing an XCD's L2 are
//     neighbours in the swizzled order.  This only permutes workgroups
//     inside a wave.
//   * 4 waves in a 2 x 2 grid, one per SIMD, each owning a (BM/2) x (BN/2)
//     sub-tile; the 256 x 128 tile runs 8 waves in a 4 x 2 grid instead, two
//     per SIMD with a 64 x 64 sub-tile each (192 registers a wave), so that
//     while one wave waits on its LDS reads or the slice barrier the other
//     keeps the matrix pipe busy, and 128 registers per SIMD stay free for
//     the consumer's waves; the 256 x 256 tile runs 8 waves in a 2 x 4 grid,
//     128 x 64 each (232 registers a wave, 48 per SIMD left for a small
//     wave beside them).  Sub-tiles are made of 16 x 16 blocks computed
//     with v_mfma_f32_16x16x32 on the 256 x 128 tile, of 32 x 32 blocks
//     computed with v_mfma_f32_32x32x16 elsewhere.
//     A and B fragments are passed to the MFMA swapped (B as the first
//     operand) so that every lane ends up with 4 consecutive columns of one
//     output row, which the epilogue writes as 8-byte pieces.
//   * K-slices of BK = 64: A and B K-slices go from memory straight into LDS
//     (gfx950 buffer loads with the LDS destination, 16 bytes per lane),
//     through a ring of LDS stages (three; six for 64 x 64 tiles, which have
//     little arithmetic per slice to hide a load behind; two 64 KiB stages
//     for 256 x 256, whose slice holds enough arithmetic to cover the next
//     slice's loads): slice k+NS-1 is loaded while slice k is multiplied, its
//     DMA instructions spread over the slice's k-steps (with two stages, all
//     at its start, so they have the whole slice to land) so the wave never
//     waits on a full memory queue with the matrix pipe idle; no VGPRs or
//     ds_write instructions are spent on staging.
//   * LDS rows are BK * 2 bytes; 16-byte chunk c of row r is stored at chunk
//     c ^ ((r / WR) % CHUNKS), WR rows sharing one 256-byte window of the 64
//     banks (BK = 64: c ^ ((r / 2) % 8)).  gfx950's LDS serves 16 lanes of a
//     ds_read_b128 per cycle over 64 banks (256 bytes): the 16 lanes read the
//     same K-chunk of 16 consecutive rows, which this swizzle spreads over all
//     64 banks.  A DMA load writes lane l's 16 bytes at position l of the
//     wave's 1 KiB destination, so each lane fetches the global chunk that
//     belongs at its position.
//   * The MFMA accumulators live in the accumulation registers (AGPRs) on
//     the four-wave tiles and in ordinary VGPRs on the eight-wave ones
//     (below); the LDS reads of k-step s+1 are issued between the MFMAs of
//     k-step s.
//   * Each wave waits for its own loads of slice k, then the workgroup meets
//     at a bare barrier (no memory-model fence, which would drain every
//     outstanding load); compiler-only fences keep LDS accesses on their side
//     of it.
//   * Global loads are buffer loads against a per-tile resource whose size
//     ends at the tile's last valid row, so rows past an edge read zeros and
//     never touch memory outside the problem.
//   * Epilogue: accumulators -> 16-bit -> LDS staging tile; every valid row's
//     destination offset (row-major, banded or subtoken layout) is computed
//     once into LDS; then 16-byte coalesced buffer stores, written through
//     the L2 (system-scope cache policy).  Once every wave has read
//     the staging tile, the workgroup issues the next tile's first NS-1
//     K-slices.  With signaling on, each wave then waits for all its memory
//     operations to complete (the tile's stores were written through the L2,
//     so complete means visible to device-coherent loads), the workgroup
//     meets at a barrier, and one lane increments cnt[group]; the lane that
//     brings it to epoch * |G_group| stores flag[group] = epoch with release
//     semantics.  The signal's waits thus overlap the next tile's first
//     loads.  With epoch stamps on, that lane first stores the epoch into the
//     slot's stamp the same way, so a consumer can check what it was shown.
//   * A third instantiation serializes the waves for tests and traces (a
//     device-wide barrier and a snapshot of the signal words after every
//     wave, cooperative launch); the hot path never runs it.
#include <type_traits>

#include "../fo_internal.h"
#include "buffer.h"

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

constexpr int kVmcntZero = 0x0F70;              // s_waitcnt vmcnt(0), other counters unconstrained
constexpr int kLgkmcntZero = 0xC07F;            // s_waitcnt lgkmcnt(0), other counters unconstrained
// Cache policy of the output stores: system scope (sc0 | sc1), i.e. written
// through the L2 to the device's point of coherence.  A finished tile is then
// visible on every XCD once its stores are complete, so it is counted without
// an L2 write-back (which cost 5-9% of the signaling GEMM on the shapes with
// short K, one per tile).
constexpr int kStoreSys = 0x11;

// s_waitcnt immediate for vmcnt(n) with the other counters unconstrained (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }

// Wait until at most min(s, S) K-slices of LOADS loads each are still in
// flight (s is wave-uniform; the waits need immediates, hence the chain).
template <int LOADS, int S>
__device__ __forceinline__ void wait_slices(int s) {
  if constexpr (S > 0) {
    if (s >= S) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(S * LOADS));
      return;
    }
    wait_slices<LOADS, S - 1>(s);
  } else {
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier that does not wait for outstanding memory operations.
__device__ __forceinline__ void bare_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One MFMA on an MB x MB output block: v_mfma_f32_32x32x16 (MB = 32, 16 fp32
// results per lane) or v_mfma_f32_16x16x32 (MB = 16, 4 per lane); both take
// 8 16-bit values of K per lane and operand.
template <int MB>
struct Acc;
template <>
struct Acc<32> { typedef f32x16 type; };
template <>
struct Acc<16> { typedef f32x4 type; };

template <typename T, int MB>
__device__ __forceinline__ typename Acc<MB>::type mma(u32x4 a, u32x4 b, typename Acc<MB>::type c);
template <>
__device__ __forceinline__ f32x16 mma<__bf16, 32>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mma<_Float16, 32>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma<__bf16, 16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mma<_Float16, 16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// Part PART of a K-slice's LDS-DMA loads: up to DPB consecutive instructions
// of the thread's A_PER_T (A rows) then B_PER_T (B rows).  Lane l of
// instruction q lands at LDS offset dst + q' * NW KiB + 16 l of its operand's
// region (NW waves per workgroup, each wave 1 KiB of every instruction).
template <int PART, int DPB, int A_PER_T, int B_PER_T, int NW>
__device__ __forceinline__ void dma_part(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, char *dst,
                                         uint32_t b_region, uint32_t g_base, uint32_t g_step, uint32_t soff) {
  constexpr int q0 = PART * DPB, q1 = q0 + DPB < A_PER_T + B_PER_T ? q0 + DPB : A_PER_T + B_PER_T;
#pragma unroll
  for (int q = q0; q < (q1 < A_PER_T ? q1 : A_PER_T); ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(dst + q * NW * 1024), 16, g_base + q * g_step, soff,
                                             0, 0);
#pragma unroll
  for (int q = (q0 > A_PER_T ? q0 : A_PER_T); q < q1; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(dst + b_region + (q - A_PER_T) * NW * 1024), 16,
                                             g_base + (q - A_PER_T) * g_step, soff, 0, 0);
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
  uint32_t c_bytes;        // size of C (at most 2^31 bytes: the plan keeps M * N <= 2^30)
  const TileDesc *slots;
  int32_t NT, W, K, remap;
  int64_t b_stride;        // elements between consecutive problems' B
  Layout L;
  uint32_t *cnt;           // NULL: no signaling
  uint32_t *flag;
  const int32_t *thr;      // |G_j|
  uint64_t *trace;
  uint32_t *stamps;        // NULL, or one word per slot: the epoch, once the slot's tile is stored
  uint32_t epoch;
  uint32_t fire_mult;      // group g fires when its counter reaches fire_mult * |G_g| (epoch, or 1 when
                           // the counters were cleared for this launch)
  int32_t P;
  uint32_t *serial;        // serialized waves only: snapshots [T][2P], then barrier counter, then status
  uint64_t timeout_ticks;  // serialized waves only: bound on one barrier wait
};

// Slot i of the plan's slot table.  The table is read-only while a kernel runs
// and a slot's index is the same for the whole workgroup, so it is read
// through the constant address space: scalar loads, counted apart from the
// vector memory operations, so fetching the next tile's descriptor does not
// wait for the previous tile's stores to complete (a vector load would: the
// wait for it counts them too).
__device__ __forceinline__ TileDesc load_slot(const TileDesc *slots, int i) {
  typedef const __attribute__((address_space(4))) TileDesc ConstTileDesc;
  const ConstTileDesc &s = ((const ConstTileDesc *)slots)[i];
  TileDesc t;
  t.row0 = s.row0;
  t.col0 = s.col0;
  t.rows = s.rows;
  t.cols = s.cols;
  t.problem = s.problem;
  t.group = s.group;
  t.base = s.base;
  t.band_stride = s.band_stride;
  return t;
}

// Device-wide barrier number k of a cooperative launch: every workgroup arrives
// once per barrier, so the k-th completes when the arrival count reaches
// (k + 1) * gridDim.x.  The wait is bounded by the device wall clock: past the
// bound (or once another workgroup has given up) the status word records
// FO_ERR_TIMEOUT and every workgroup leaves.  Returns false on a time-out.
__device__ __forceinline__ bool grid_barrier(uint32_t *bar, uint32_t *status, uint32_t k, uint64_t timeout) {
  __shared__ int s_ok;
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = 1;
    __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t target = (k + 1u) * gridDim.x;
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 || wall_clock64() - t0 > timeout) {
        uint32_t expected = 0;
        __hip_atomic_compare_exchange_strong(status, &expected, (uint32_t)FO_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0;
}

// After wave `w` of a serialized launch: all workgroups meet, workgroup 0
// copies cnt[P] then flag[P] into snapshot w, and a second barrier keeps every
// workgroup out of wave w+1 until the copy is taken.
__device__ __forceinline__ bool wave_snapshot(const GemmParams &p, int w) {
  const int T = (p.NT + p.W - 1) / p.W;
  uint32_t *bar = p.serial + 2 * (int64_t)T * p.P, *status = bar + 1;
  if (!grid_barrier(bar, status, 2u * w, p.timeout_ticks)) return false;
  if (blockIdx.x == 0) {
    uint32_t *snap = p.serial + 2 * (int64_t)w * p.P;
    for (int i = threadIdx.x; i < p.P; i += blockDim.x) {
      snap[i] = __hip_atomic_load(&p.cnt[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      snap[p.P + i] = __hip_atomic_load(&p.flag[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  return grid_barrier(bar, status, 2u * w + 1u, p.timeout_ticks);
}

// Tile BM x BN, K-slices of BK = 64 staged in LDS, NW waves per workgroup
// (4: one per SIMD; 8: two per SIMD) in a WGM x WGN grid.
template <int BM, int BN, int BK, int NW>
struct Cfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int WGM = NW == 4 ? 2 : (BM == BN ? 2 : 4);
  static constexpr int WGN = NW / WGM;
  static constexpr int ROWB = BK * 2;                 // bytes of one staged row of A or B
  static constexpr int CHUNKS = BK / 8;               // 16-byte chunks per staged row
  // MFMA block: 16 x 16 x 32 on the 256 x 128 tile -- under the power cap the
  // matrix pipe sustains about 13% more FLOP/s with it than with 32 x 32 x 16
  // on the same values when two waves share a SIMD, each with a 4 x 4 block
  // grid (the tile ran 9-11% faster) -- and 32 x 32 x 16 elsewhere: one wave
  // per SIMD (the four-wave tiles) leaves the smaller instruction's
  // accumulation chains too short to cover its latency (the 128 x 128 tile
  // ran 16% slower with it), and on the 256 x 256 tile the fragments of two
  // k-steps of 16 x 16 blocks take twice the registers: a wave would hold all
  // 256, leaving no room on the SIMD for another wave beside the GEMM.
  static constexpr int MB = NW == 8 && BN == 128 ? 16 : 32;
  static constexpr int LG = 64 / MB;                  // lane groups: lanes l, l + MB, ... hold successive K-chunks
  static constexpr int KS = BK / (8 * LG);            // MFMA k-steps per slice (each 8 * LG deep)
  static constexpr int GPB = MB * MB / 256;           // groups of 4 output columns a lane holds per block
  static constexpr int RPK = 1024 / ROWB;             // staged rows per KiB (one DMA instruction of a wave)
  static constexpr int WR = 256 / ROWB;               // rows that share one 256-byte window of the 64 banks
  // LDS ring depth: slice k+NS-1 is loaded while slice k is multiplied.  Small
  // tiles have little arithmetic per slice, so they keep more slices in flight;
  // two 64 KiB stages of the 256 x 256 tile fill the LDS.
  static constexpr int NS = BM == 64 ? 6 : (BM == 256 && BN == 256 ? 2 : 3);
  // Accumulators in ordinary VGPRs (the eight-wave tiles): with two waves per
  // SIMD a wave has 256 registers, which in the accumulation-register form the
  // compiler splits evenly (accumulators + the rest, each at most 128: the
  // fragments then spilled into the accumulation registers, or to memory); in
  // the VGPR form the accumulators and the rest share one budget.
  static constexpr bool VGPR_ACC = NW == 8;
  static constexpr int DIST = NS - 1;                 // prefetch distance in slices
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / MB, FN = WN / MB;
  static constexpr int A_PER_T = BM * CHUNKS / THREADS;  // 16-byte chunks per thread per stage
  static constexpr int B_PER_T = BN * CHUNKS / THREADS;
  static constexpr int LOADS = A_PER_T + B_PER_T;     // DMA instructions per thread per stage
  // of them issued per k-step (fewer in the last parts); with two stages, all in the first
  static constexpr int DPB = NS == 2 ? LOADS : (LOADS + KS - 1) / KS;
  static constexpr int STAGE = (BM + BN) * ROWB;
  static constexpr int OUT_PITCH = BN * 2 + 16;      // bytes per staged output row
  static constexpr int OUT_BYTES = BM * OUT_PITCH;
  static constexpr int ROWOFF = OUT_BYTES;           // int64 per row after the staging tile
  static constexpr int LDS = (NS * STAGE > OUT_BYTES + BM * 8) ? NS * STAGE : OUT_BYTES + BM * 8;
  static_assert(BK == 64, "slice depth");
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  static_assert(BM * CHUNKS % THREADS == 0 && BN * CHUNKS % THREADS == 0, "chunk split");
  static_assert(FM >= 1 && FN >= 1 && WM % MB == 0 && WN % MB == 0, "wave tile");
  static_assert(NS * LOADS <= 63, "loads in flight fit the vmcnt counter");
  static_assert(LDS <= 160 * 1024, "LDS of one CU");
};

// Calls f(integral_constant<I>) ... f(integral_constant<N-1>): the k-steps of a
// slice, each with its own compile-time part of the slice's loads.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// SIGNAL: the signaling GEMM (reordered stores, counting table, flags); otherwise
// the plain GEMM with a row-major epilogue.  Separate instantiations keep the
// plain kernel free of signaling code and give the two distinct symbols.
// SERIAL (with SIGNAL, cooperative launch only): a device-wide barrier after
// every wave and a snapshot of the signal words, so that the waves are
// physical and each wave's counting table can be read back; every workgroup
// then runs exactly T iterations, idling through the tile work of a partial
// last wave.
// SKIP (plans with ragged tiles only): a wave whose part of the tile lies
// wholly past its edge skips its fragment reads and MFMAs; a separate
// instantiation, so full-tile plans run code without the branch.
template <typename T, int BM, int BN, int BK, int NW, bool SIGNAL, bool SERIAL, bool SKIP>
__global__ __launch_bounds__(64 * NW, 1) void gemm_kernel(GemmParams p) {
  using C = Cfg<BM, BN, BK, NW>;
  constexpr int kRowBytes = C::ROWB;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // Naming an accumulation register here lets the compiler give the MFMAs
  // their accumulation-register form, so the accumulators live outside the
  // 256 architectural VGPRs that the operands, offsets and addresses need
  // (not with VGPR_ACC: 232 registers in one budget, no spills, against
  // 128 + 128 and spills in the split form).
#if defined(__HIP_DEVICE_COMPILE__)  // the register name exists only for the GPU target
  if constexpr (!C::VGPR_ACC) asm volatile("; accumulators in AGPRs" ::: "a0");
#endif
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS destinations go to M0
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int g = blockIdx.x;
  const int pos = p.remap ? (g & 7) * (p.W >> 3) + (g >> 3) : g;
  const int nk = p.K / BK;
  const uint32_t row_bytes = (uint32_t)p.K * 2u;

  // LDS rows hold CHUNKS 16-byte chunks; chunk c of row r is stored at physical
  // chunk c ^ ((r / WR) % CHUNKS), WR rows filling one 256-byte window of the
  // 64 banks: the 16 lanes a ds_read_b128 serves per cycle read one logical
  // chunk of 16 consecutive rows, which this spreads over all 64 banks (BK = 64:
  // 2 rows per window, XOR over 8 chunks).
  // global -> LDS coordinates.  DMA instruction i of wave w fills 1 KiB of
  // LDS: rows (NW i + w) * RPK .. + RPK of the operand.  Lane l lands at
  // physical chunk l % CHUNKS of row r = (NW i + w) * RPK + l / CHUNKS, which
  // holds logical chunk (l % CHUNKS) ^ ((r / WR) % CHUNKS); NW RPK / WR is a
  // multiple of CHUNKS, so row and chunk depend on i only through a stride.
  const int dma_row = wave * C::RPK + lane / C::CHUNKS;
  const uint32_t g_base = (uint32_t)dma_row * row_bytes +
                          (uint32_t)(((lane % C::CHUNKS) ^ ((dma_row / C::WR) % C::CHUNKS)) << 4);
  const uint32_t g_step = (uint32_t)NW * C::RPK * row_bytes;
  static_assert((NW * C::RPK / C::WR) % C::CHUNKS == 0, "the swizzle repeats every NW RPK rows");
  constexpr uint32_t s_bofs = BM * kRowBytes;      // B rows follow A rows in a stage
  // MFMA fragment reads: row (lane % MB) of each MB-row block, K-chunk ks * LG + lane / MB
  const int frag_row = lane % C::MB, frag_g = lane / C::MB, swz = (frag_row / C::WR) % C::CHUNKS;
  static_assert((C::MB / C::WR) % C::CHUNKS == 0, "every block of MB rows has the same swizzle");
  const uint32_t a_frag = (uint32_t)((wm * C::WM + frag_row) * kRowBytes);
  const uint32_t b_frag = (uint32_t)(s_bofs + (wn * C::WN + frag_row) * kRowBytes);

  int64_t *rowoff = reinterpret_cast<int64_t *>(smem + C::ROWOFF);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C, p.c_bytes);

  // The tile a workgroup works on and its buffer resources.  A tile's first
  // NS-1 K-slices are issued as soon as the previous tile's staging area is
  // free, before that tile's signal, so the signal's waits overlap them.
  TileDesc t = load_slot(p.slots, 0);
  __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, 0), rb = make_rsrc(p.B, 0);
  auto load_tile = [&](int bb) {
    t = load_slot(p.slots, bb);
    ra = make_rsrc(p.A + (int64_t)t.row0 * p.K, t.rows * row_bytes);
    rb = make_rsrc(p.B + (int64_t)t.problem * p.b_stride + (int64_t)t.col0 * p.K, t.cols * row_bytes);
  };
  // K-slice kt -> LDS stage kt % NS, as C::LOADS DMA instructions per thread;
  // part p of KS (one per k-step) issues instructions [p * DPB, (p + 1) * DPB)
  constexpr int DPB = C::DPB;
  auto stage_dst = [&](int kt) { return smem + (kt % C::NS) * C::STAGE + wave * 1024; };
#define FO_DMA_PART(PART, KT)                                                                              \
  dma_part<PART, DPB, C::A_PER_T, C::B_PER_T, NW>(ra, rb, stage_dst(KT), s_bofs, g_base, g_step,          \
                                                  (uint32_t)(KT) * kRowBytes)
  auto issue = [&](int kt) {
    static_for<0, C::KS>([&](auto part) { FO_DMA_PART(decltype(part)::value, kt); });
  };
  auto prologue = [&]() {  // slices 0 .. NS-2 of the current tile
#pragma unroll
    for (int kt = 0; kt < C::DIST; ++kt)
      if (kt < nk) issue(kt);
  };
  if (pos < p.NT) {
    load_tile(pos);
    prologue();
  }

  const int iters = SERIAL ? (p.NT + p.W - 1) / p.W : 0;
  for (int b = pos, it = 0; SERIAL ? it < iters : b < p.NT; b += p.W, ++it) {
    if (SERIAL && b >= p.NT) {  // no tile in this (partial) wave: only the barriers
      if (!wave_snapshot(p, it)) return;
      continue;
    }

    typename Acc<C::MB>::type acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = typename Acc<C::MB>::type{};

    // Fragments of one k-step of a stage, into register set u, read
    // in the order the MFMAs below consume them.
    u32x4 fa[2][C::FM], fb[2][C::FN];
    auto read_frags = [&](int u, int stage, int ks) {
      const char *base = smem + (stage % C::NS) * C::STAGE;
      const uint32_t chunk = (uint32_t)(((ks * C::LG + frag_g) ^ swz) << 4);
      fa[u][0] = *reinterpret_cast<const u32x4 *>(base + a_frag + chunk);
#pragma unroll
      for (int f = 0; f < C::FN; ++f)
        fb[u][f] = *reinterpret_cast<const u32x4 *>(base + b_frag + f * C::MB * kRowBytes + chunk);
#pragma unroll
      for (int f = 1; f < C::FM; ++f)
        fa[u][f] = *reinterpret_cast<const u32x4 *>(base + a_frag + f * C::MB * kRowBytes + chunk);
    };
    auto mfmas = [&](int u) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mma<T, C::MB>(fb[u][j], fa[u][i], acc[i][j]);
    };
    // Order inside a block: its share of DMA loads spread out, its LDS reads
    // alternating with its MFMAs, so the wave never sits on a queue while the
    // matrix pipe has nothing to do.
    constexpr int NR = C::FM + C::FN, NM = C::FM * C::FN;
    auto block_order_dma = [&](auto nd) {  // nd: this block's DMA instructions
      constexpr int ND = decltype(nd)::value;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r % 2 == 0 && r / 2 < ND) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                // DS read
        if (r < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
      }
      if ((NR + 1) / 2 < ND) __builtin_amdgcn_sched_group_barrier(0x020, ND - (NR + 1) / 2, 0);
      if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto block_order = [&]() {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (r < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
      __builtin_amdgcn_sched_barrier(0);
    };

    // Stage s % NS holds slice s from when it is loaded (during slice s-D, D =
    // NS-1) until its last fragments are read (k-step KS-1 of slice s).  Slice
    // kt+D's loads are spread over the KS blocks of slice kt.  Slices
    // 0 .. D-1 were issued ahead (prologue); anything this wave issued before
    // them (the previous tile's stores) is older, so the same counts hold:
    // slice 0 has landed once at most min(D-1, nk-1) slices are in flight.
    // Block s of a slice reads the fragments of k-step s+1 while the MFMAs of
    // k-step s run; the last block hands over to the next slice.
    constexpr int D = C::DIST, KS = C::KS, LAST = (KS - 1) % 2;
    wait_slices<C::LOADS, D - 1>(nk - 1);
    bare_barrier();
    // With SKIP, a wave whose rows or columns of the tile lie wholly past its
    // edge (an expert's last, mostly empty tile row) has nothing to multiply:
    // it runs the second loop below, the same loads, waits and barriers in the
    // same order (its loads fill LDS for the other waves) without fragment
    // reads or MFMAs, so its SIMD's matrix pipe serves the other wave of the
    // pair alone.  Without SKIP the condition is a constant and only the first
    // loop exists.  wm, wn and the tile's extent are the same in every lane.
    bool multiplies = true;
    if constexpr (SKIP) multiplies = wm * C::WM < t.rows && wn * C::WN < t.cols;
    if (multiplies) {
      read_frags(0, 0, 0);
      // The last slice is peeled off so that the loop body has no join point at
      // which the wait-count insertion would have to assume the worst of two paths.
      auto blocks_dma = [&](int kt) {  // blocks 0 .. KS-2, with parts 0 .. KS-2 of slice kt+D's loads
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, KS - 1>([&](auto sc) {
          constexpr int st = decltype(sc)::value;
          constexpr int left = C::LOADS - st * DPB;
          FO_DMA_PART(st, kt + D);
          read_frags((st + 1) % 2, kt, st + 1);
          mfmas(st % 2);
          block_order_dma(std::integral_constant<int, (left < 0 ? 0 : left < DPB ? left : DPB)>{});
        });
      };
      auto blocks = [&](int kt) {
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, KS - 1>([&](auto sc) {
          constexpr int st = decltype(sc)::value;
          read_frags((st + 1) % 2, kt, st + 1);
          mfmas(st % 2);
          block_order();
        });
      };
      // Steady state: one path per iteration, so the accumulators keep their
      // registers from one iteration to the next.
      int kt = 0;
      for (; kt + D < nk; ++kt) {
        blocks_dma(kt);
        FO_DMA_PART(KS - 1, kt + D);
        // this wave's reads of slice kt are complete and its loads of slice kt+1
        // landed (slices kt+2 .. kt+D may still be in flight)
        __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 1) * C::LOADS));
        bare_barrier();  // no wave reads slice kt any more; slice kt+1 is in LDS for every wave
        read_frags(0, kt + 1, 0);
        mfmas(LAST);
        block_order();
      }
      // the last handovers: nothing left to load, slices kt+2 .. nk-1 in flight
      auto drain = [&](int kt) {
        blocks(kt);
        __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
        wait_slices<C::LOADS, D - 2>(nk - 2 - kt);
        bare_barrier();
        read_frags(0, kt + 1, 0);
        mfmas(LAST);
        block_order();
      };
      if constexpr (D == 2) {
        if (kt + 1 < nk) drain(kt++);
      } else {
        for (; kt + 1 < nk; ++kt) drain(kt);
      }
      blocks(nk - 1);
      mfmas(LAST);
    } else {
      // the barrier skeleton of the loop above: slice kt+D's loads (all KS
      // parts) during slice kt, then the same waits and one barrier per slice
      int kt = 0;
      for (; kt + D < nk; ++kt) {
        static_for<0, KS>([&](auto part) { FO_DMA_PART(decltype(part)::value, kt + D); });
        __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 1) * C::LOADS));
        bare_barrier();
      }
      auto drain_idle = [&](int kt) {
        wait_slices<C::LOADS, D - 2>(nk - 2 - kt);
        bare_barrier();
      };
      if constexpr (D == 2) {
        if (kt + 1 < nk) drain_idle(kt++);
      } else {
        for (; kt + 1 < nk; ++kt) drain_idle(kt);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // all fragment reads done before the staging tile overwrites the ring

    // ---- epilogue: destination of every valid row, then the 16-bit tile through LDS
    if (tid < BM) rowoff[tid] = tid < t.rows ? row_offset(p.L, t, b, tid) : 0;
    // Every LDS address below is one per-thread base plus a compile-time offset
    // (an instruction immediate), so no per-fragment address is computed once
    // and kept in a register across tiles: on a 256 x 256 tile that alone ran
    // the VGPRs out next to 256 accumulators.
    // Lane l holds, of every block, row l % MB and the 4 consecutive columns
    // g * 4 LG + 4 (l / MB) .. + 3 for each of its GPB groups g.
    char *const stage_w = smem + (wm * C::WM + frag_row) * C::OUT_PITCH + (wn * C::WN + frag_g * 4) * 2;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
#pragma unroll
        for (int g4 = 0; g4 < C::GPB; ++g4) {
          const f32x4 v = {acc[i][j][g4 * 4 + 0], acc[i][j][g4 * 4 + 1], acc[i][j][g4 * 4 + 2], acc[i][j][g4 * 4 + 3]};
          *reinterpret_cast<u32x2 *>(stage_w + i * C::MB * C::OUT_PITCH + (j * C::MB + g4 * 4 * C::LG) * 2) =
              pack4<T>(v);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    __syncthreads();
    constexpr int CPR = BN / 8;                 // 16-byte chunks per row
    constexpr int RPI = C::THREADS / CPR;       // rows per iteration of the store loop
    static_assert(C::THREADS % CPR == 0 && BM % RPI == 0, "whole rows per iteration");
    const int r_t = tid / CPR, c8 = tid % CPR;  // a thread's row in each block of RPI rows, and its chunk
    const char *const stage_r = smem + r_t * C::OUT_PITCH + c8 * 16;
    const int64_t *const rowoff_t = rowoff + r_t;
    const bool col_ok = c8 * 8 < t.cols;
#pragma unroll
    for (int i = 0; i < BM / RPI; ++i) {
      if (r_t + i * RPI < t.rows && col_ok) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(stage_r + i * RPI * C::OUT_PITCH);
        __builtin_amdgcn_raw_buffer_store_b128(v, rc, (uint32_t)rowoff_t[i * RPI] * 2u + (uint32_t)c8 * 16u, 0,
                                               kStoreSys);
      }
    }

    // ---- next tile: once every wave has read the staging tile and the row
    // offsets, its first slices may overwrite them.
    __syncthreads();
    const int grp = t.group;
    const bool more = b + p.W < p.NT;
    if (more) {
      load_tile(b + p.W);
      prologue();
    }

    // ---- signal: counting table, then the group's flag.  The tile's stores
    // went out with the system-scope cache policy, i.e. written through the
    // L2 to the device's point of coherence, and such a store counts as
    // complete only once the memory side has taken it.  So each wave waits
    // until every memory operation it issued is complete (its stores, and the
    // next tile's first slices issued after them: the ISA does not order a
    // store's completion with younger loads), the workgroup meets at a
    // barrier, and the whole tile is then visible to device-coherent loads on
    // every XCD without an L2 write-back.  One lane counts the tile; the lane
    // that completes the group raises the flag with a release store.
    if constexpr (SIGNAL) {
      __builtin_amdgcn_s_waitcnt(kVmcntZero);
      __syncthreads();
      if (tid == 0) {
        if (p.stamps) {  // device scope, written through like the tile; complete before the tile is counted
          __hip_atomic_store(&p.stamps[b], p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_s_waitcnt(kVmcntZero);
        }
        const uint32_t old = __hip_atomic_fetch_add(&p.cnt[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool fire = old + 1u == p.fire_mult * (uint32_t)p.thr[grp];
        if (fire) __hip_atomic_store(&p.flag[grp], p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        if (p.trace) {
          p.trace[2 * (int64_t)b] = wall_clock64();
          p.trace[2 * (int64_t)b + 1] = ((uint64_t)(uint32_t)g << 32) | old;
          if (fire) __hip_atomic_fetch_add(&p.trace[2 * (int64_t)p.NT + grp], (uint64_t)1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if constexpr (SERIAL) {
      if (!wave_snapshot(p, it)) return;
    }
  }
#undef FO_DMA_PART
}

template <typename T, int BM, int BN, int BK, int NW, bool SIGNAL, bool SERIAL, bool SKIP = false>
int launch_typed(const fo_plan *pl, const GemmParams &gp, hipStream_t s) {
  using C = Cfg<BM, BN, BK, NW>;
  const void *fn = reinterpret_cast<const void *>(&gemm_kernel<T, BM, BN, BK, NW, SIGNAL, SERIAL, SKIP>);
  static bool configured = false;  // per process; the attribute is per kernel and device-independent
  if (!configured) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS) != hipSuccess) return FO_ERR_HIP;
    configured = true;
  }
  if constexpr (SERIAL) {
    // every workgroup must be resident at once, or the barriers could not complete
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, C::THREADS, C::LDS) != hipSuccess)
      return FO_ERR_HIP;
    if ((int64_t)per_cu * pl->num_cus < gp.W) return FO_ERR_UNSUPPORTED;
    GemmParams arg = gp;
    void *args[] = {&arg};
    if (hipLaunchCooperativeKernel(fn, dim3(gp.W), dim3(C::THREADS), args, C::LDS, s) != hipSuccess)
      return FO_ERR_HIP;
    return FO_OK;
  } else {
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, NW, SIGNAL, false, SKIP>), dim3(gp.W), dim3(C::THREADS), C::LDS, s,
                       gp);
    return hipGetLastError() == hipSuccess ? FO_OK : FO_ERR_HIP;
  }
}

template <typename T, int BM, int BN, bool SIGNAL, bool SERIAL>
int launch_8wave(const fo_plan *p, const GemmParams &gp, hipStream_t s) {
  using C8 = Cfg<BM, BN, 64, 8>;
  if constexpr (!SERIAL) {
    if (p->min_tile_rows <= BM - C8::WM || p->min_tile_cols <= BN - C8::WN)
      return launch_typed<T, BM, BN, 64, 8, SIGNAL, SERIAL, true>(p, gp, s);
  }
  return launch_typed<T, BM, BN, 64, 8, SIGNAL, SERIAL>(p, gp, s);
}

template <typename T, bool SIGNAL, bool SERIAL>
int launch_tile(const fo_plan *p, const GemmParams &gp, hipStream_t s) {
  // The eight-wave tiles share each SIMD between two waves: on a plan with a
  // tile whose wave band (rows or columns) lies wholly past its edge, the
  // band's waves skipping their MFMAs lets the other wave of each pair run
  // alone (the four-wave tiles, one wave per SIMD, gain nothing from it).
  if (p->BM == 256 && p->BN == 256) return launch_8wave<T, 256, 256, SIGNAL, SERIAL>(p, gp, s);
  if (p->BM == 256 && p->BN == 128) return launch_8wave<T, 256, 128, SIGNAL, SERIAL>(p, gp, s);
  if (p->BM == 128 && p->BN == 128) return launch_typed<T, 128, 128, 64, 4, SIGNAL, SERIAL>(p, gp, s);
  if (p->BM == 64 && p->BN == 64) return launch_typed<T, 64, 64, 64, 4, SIGNAL, SERIAL>(p, gp, s);
  return FO_ERR_UNSUPPORTED;
}

}  // namespace

int launch_gemm(const fo_plan *p, const void *A, const void *B, void *Cout, bool rowmajor, uint32_t *sig,
                uint32_t epoch, uint64_t *trace, uint32_t *serial, hipStream_t s, bool counts_cleared) {
  if (p->NT == 0) return FO_OK;
  GemmParams gp{};
  gp.A = static_cast<const uint16_t *>(A);
  gp.B = static_cast<const uint16_t *>(B);
  gp.C = static_cast<uint16_t *>(Cout);
  gp.c_bytes = (uint32_t)(2 * p->M * p->N);
  gp.slots = p->d_slots;
  gp.NT = p->NT;
  gp.W = p->W;
  gp.K = (int32_t)p->K;
  gp.remap = (p->W % 8 == 0) ? 1 : 0;
  gp.b_stride = p->N * p->K;
  gp.L = p->layout(true);
  if (rowmajor) gp.L.mode = kRowMajor;
  gp.cnt = sig;
  gp.flag = sig ? sig + p->flag_offset() : nullptr;
  gp.thr = p->d_group_tiles;
  gp.trace = sig ? trace : nullptr;
  gp.stamps = sig && p->stamps() ? sig + p->stamp_offset() : nullptr;
  gp.epoch = epoch;
  gp.fire_mult = counts_cleared ? 1u : epoch;
  gp.P = p->P;
  gp.serial = serial;
  gp.timeout_ticks = 2000000ull * p->ticks_per_us;  // 2 s per barrier wait
  const bool bf = p->dtype == FO_BF16;
  if (serial) {
    if (!gp.cnt) return FO_ERR_INVALID;
    return bf ? launch_tile<__bf16, true, true>(p, gp, s) : launch_tile<_Float16, true, true>(p, gp, s);
  }
  if (gp.cnt) return bf ? launch_tile<__bf16, true, false>(p, gp, s) : launch_tile<_Float16, true, false>(p, gp, s);
  return bf ? launch_tile<__bf16, false, false>(p, gp, s) : launch_tile<_Float16, false, false>(p, gp, s);
}

}  // namespace fo
