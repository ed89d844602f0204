/*
 * fo.h -- C ABI of the signaling GEMM with tile reordering for AMD MI355X (gfx950).
 *
 * The method is FlashOverlap's hot path, as the deep-dive page
 * "FlashOverlap: 信号驱动计算通信重叠论文详解" (cited below as "deep-dive") and
 * the summary page "Efficient and Adaptable Overlapping for Computation and
 * Communication via Signaling and Reordering" (cited as "summary") describe it:
 *
 *   - one uninterrupted GEMM kernel (deep-dive, 核心设计 › 计算侧);
 *   - its epilogue writes every finished tile through a mapping table into a
 *     contiguous span per wave group (deep-dive 二、重排机制 › 解决方案),
 *     then adds one to the group's entry of a counting table and raises the
 *     group's signal when the entry reaches |G_j| (deep-dive 一、信号机制 ›
 *     实现方法: 组级 Tile 计数; 五、CUTLASS 扩展实现 › 扩展主循环);
 *   - a second kernel on another stream watches the signals and handles each
 *     group's span as soon as it is signalled (deep-dive 五 › 专用监控内核;
 *     核心设计 › 通信侧).  On one GPU it reduces the span with a second
 *     buffer, a local stand-in for the group's collective;
 *   - a post-communication kernel applies the inverse mapping and restores
 *     row-major layout (deep-dive 二 › 解决方案; summary, Figure 5).
 *
 * Conventions shared by every call
 *   - Return value: FO_OK (0) or a negative fo_status.  No call throws.
 *   - Device pointers must be 16-byte aligned; host arrays have no alignment
 *     requirement.  The caller allocates and owns every buffer it passes.
 *   - Enqueue calls (fo_gemm_*, fo_consume_group, fo_reorder_*) are
 *     asynchronous on the given HIP stream; they neither allocate nor copy
 *     from the host nor synchronise.  Errors they return are detected on the
 *     host before any launch; errors that arise on the device are written to
 *     a caller-provided status word.  They need the plan's device to be the
 *     current HIP device (FO_ERR_INVALID otherwise), and the stream and
 *     buffers to belong to it.
 *   - Element types: FO_BF16 or FO_FP16 for A, B and every output buffer.
 *     Accumulation is fp32; results are rounded to the element type,
 *     round-to-nearest-even.
 */
#ifndef FO_H_
#define FO_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fo_status {
  FO_OK = 0,
  FO_ERR_INVALID = -1,      /* bad argument: null or misaligned pointer, bad sizes, bad partition */
  FO_ERR_UNSUPPORTED = -2,  /* valid request the library does not implement (e.g. K % 64 != 0)*/
  FO_ERR_HIP = -3,          /* a HIP runtime call failed                                       */
  FO_ERR_NOMEM = -4,        /* host or device allocation failed at plan creation               */
  FO_ERR_TIMEOUT = -5,      /* device-side: the consumer waited longer than its time limit     */
  FO_ERR_STALE = -6         /* device-side: with FO_PLAN_EPOCH_STAMPS, the consumer read a
                               tile stamp of an older epoch after its group's signal          */
} fo_status;

typedef enum fo_dtype { FO_BF16 = 0, FO_FP16 = 1 } fo_dtype;

/* Reorder pattern per collective (deep-dive 二 › 不同通信原语的重排模式, Figure 6). */
typedef enum fo_mode {
  FO_MODE_TILE = 0,      /* AllReduce: whole tiles, row-major inside the tile             */
  FO_MODE_SUBTILE = 1,   /* ReduceScatter: each tile cut into `ranks` row bands; a group's
                            span holds band k of all its tiles as rank segment k           */
  FO_MODE_SUBTOKEN = 2   /* All-to-All: each tile row goes to the bucket of its row's
                            destination; a group's span holds `ranks` buckets              */
} fo_mode;

/* Element-wise activation of the fused post-reorder epilogue. */
typedef enum fo_act {
  FO_ACT_NONE = 0,
  FO_ACT_RELU = 1,   /* max(x, 0)            */
  FO_ACT_SILU = 2,   /* x / (1 + exp(-x))    */
} fo_act;

/* Storage of B.  Only FO_B_NK is implemented: a plan asking for FO_B_KN is refused with
 * FO_ERR_UNSUPPORTED (the kernels stage B rows of K contiguous elements). */
typedef enum fo_b_layout {
  FO_B_NK = 0,       /* B stored [N, K], K contiguous (a linear layer's weight); the default */
  FO_B_KN = 1        /* B stored [K, N], N contiguous: not supported                         */
} fo_b_layout;

/* Plan flags. */
#define FO_PLAN_HOST_ONLY 0x1u   /* build the tables on the host only; enqueue calls reject the plan */
#define FO_PLAN_EPOCH_STAMPS 0x2u /* stale-read detector: the signal buffer grows by one word per
                                    slot (stamp_offset, fo_plan_info); the signaling GEMM writes the
                                    epoch into its tile's stamp after the tile's stores are complete
                                    and before the tile is counted, and the consumer, after a
                                    group's signal, reads every stamp of the group with the same
                                    loads it uses for the span: a stamp of an older epoch means the
                                    signal did not make the tile's writes visible, and it stores
                                    FO_ERR_STALE into its status word (it still finishes the
                                    group).  The stamps are published the same way as the data
                                    (written through the L2 and complete before the count), so
                                    they observe the protocol, not just the data               */

/*
 * Problem description.  C[M, N] = A[M, K] . B^T where B is stored [N, K]
 * (K contiguous, a linear layer's weight); A is row-major [M, K].  A grouped
 * GEMM (MoE experts) stacks the problems' rows: A is [sum m_e, K], B holds
 * num_problems consecutive [N, K] matrices, C is [sum m_e, N].
 *
 * Tiles are BM x BN; dispatch index b walks the tile grid in grouped-M
 * order of width `swizzle` (bands of `swizzle` tile rows, column by column
 * inside a band; deep-dive 一 › Block Swizzling 的影响), problem after
 * problem.  Wave w holds dispatch indices [w*W, (w+1)*W) (deep-dive 一 ›
 * 关键洞察: a wave is as many tiles as run at once); the GEMM runs a
 * persistent grid of exactly W workgroups, so wave w is each workgroup's
 * w-th tile.  T = ceil(NT / W).  The T waves are cut into P groups of
 * waves_per_group[j] consecutive waves (deep-dive 一 › Wave Group 设计,
 * 三 › 设计空间大小).  Slot s of the mapping table holds the tile with
 * dispatch index s, so each group occupies consecutive slots and one
 * contiguous span of the reordered buffer.  Edge tiles are packed.
 */
typedef struct fo_plan_desc {
  int32_t num_problems;            /* >= 1                                                    */
  const int64_t *m_per_problem;    /* host [num_problems]: rows of each problem (>= 0)        */
  int64_t N, K;                    /* N % 8 == 0, K % 64 == 0, both > 0; M*N <= 2^30; the
                                      tile's operand rows fit 32-bit byte offsets:
                                      max(BM, BN) * K * 2 < 2^32 (K < 2^23 at BM = 256)       */
  int32_t dtype;                   /* fo_dtype                                                */
  int32_t BM, BN;                  /* tile: 256x256, 256x128, 128x128 or 64x64; 0,0 = 256x128 */
  int32_t swizzle;                 /* S >= 1; 0 = 4                                           */
  int32_t wave_size;               /* W >= 1; 0 = the device's CU count (256 if host-only)    */
  int32_t num_groups;              /* P; 0 = one wave per group (waves_per_group ignored)     */
  const int32_t *waves_per_group;  /* host [P]: composition of T, every entry >= 1            */
  int32_t mode;                    /* fo_mode                                                 */
  int32_t ranks;                   /* R (SUBTILE: BM % R == 0, full tiles) or D (SUBTOKEN)    */
  const int32_t *row_dest;         /* host [M], SUBTOKEN only: destination rank of each row   */
  const int32_t *dispatch_order;   /* host [NT] or NULL: explicit b -> tile permutation       */
  uint32_t flags;                  /* FO_PLAN_* bits                                          */
  int32_t b_layout;                /* fo_b_layout; FO_B_KN -> FO_ERR_UNSUPPORTED              */
} fo_plan_desc;

typedef struct fo_plan fo_plan;

typedef struct fo_plan_info {
  int64_t M, N, K;
  int32_t BM, BN, swizzle, wave_size;
  int32_t NT;                      /* tiles                                                   */
  int32_t T;                       /* waves                                                   */
  int32_t P;                       /* groups                                                  */
  int32_t num_units;               /* consumer work units (collective calls) over all groups  */
  int32_t mode, ranks, dtype, num_problems;
  int32_t device;                  /* HIP device the tables live on; -1 if host-only          */
  int32_t clock_khz;               /* rate of the device wall clock used by the traces; 0 if host-only */
  int32_t sig_words;               /* uint32 words of the signal buffer: flag_offset + P, or
                                      stamp_offset + NT with FO_PLAN_EPOCH_STAMPS             */
  int32_t flag_offset;             /* word index of flag[0]: P rounded up to a multiple of 64 */
  int32_t stamp_offset;            /* word index of stamp[0] (slot order) with
                                      FO_PLAN_EPOCH_STAMPS, else -1                           */
  int32_t flags;                   /* the plan's FO_PLAN_* bits                               */
} fo_plan_info;

/*
 * Build a plan (deep-dive 一、信号机制 › Wave Group 设计 and 实现方法: 组级 Tile
 * 计数 for the waves, groups and thresholds; 二、重排机制 › 解决方案: 映射表重排
 * and Figure 6 for the mapping table and the three span layouts; 三、Wave Group
 * 划分设计空间 for the partition): tile grid, dispatch order, waves, groups,
 * mapping table, thresholds |G_j| (in tiles), span and unit offsets, and the
 * per-slot records the kernels read.
 *
 * Unless FO_PLAN_HOST_ONLY is set the tables are uploaded once to the current
 * HIP device (one device allocation, owned by the plan, freed by
 * fo_plan_destroy); they are immutable afterwards, so a plan may be shared by
 * streams and threads.  The plan must outlive all work enqueued with it.
 * *out is set only on FO_OK; desc and every host array it points to are
 * copied, the caller keeps them.
 *
 * Errors: FO_ERR_INVALID for a malformed description (null or negative
 * sizes, a composition that does not sum to T, an entry < 1, a row_dest out
 * of range, ReduceScatter with BM % R != 0 or a ragged tile, a dispatch order
 * that is not a permutation); FO_ERR_UNSUPPORTED for a request the kernels do
 * not implement: another tile shape, K % 64 != 0, an element type other than
 * bf16/fp16, B stored [K, N], M*N > 2^30, max(BM, BN) * K * 2 >= 2^32, or a
 * current device that is not gfx950 (fo_arch_supported); FO_ERR_HIP when the
 * runtime cannot be queried; FO_ERR_NOMEM when an allocation fails.
 */
int fo_plan_groups(const fo_plan_desc *desc, fo_plan **out);
int fo_plan_destroy(fo_plan *plan);
int fo_plan_info_get(const fo_plan *plan, fo_plan_info *out);

/*
 * 1 if a device whose gcnArchName is `arch` (e.g. "gfx950:sramecc+:xnack-")
 * can run the kernels, i.e. its processor is gfx950; 0 otherwise or for NULL.
 * fo_plan_groups applies it to the current device of a non-host-only plan.
 */
int fo_arch_supported(const char *arch);

/*
 * Copy the plan's host tables into caller arrays (any may be NULL):
 *   tile_of_slot[NT]  inverse mapping table: slot -> row-major tile index
 *                     (tiles of problem e follow those of problems < e)
 *   slot_of_tile[NT]  mapping table: tile -> slot
 *   group_of_slot[NT] group j of each slot
 *   group_tiles[P]    |G_j| in tiles: the counting table's target per group
 *   span_off[P+1]     element offset of each group's contiguous span
 */
int fo_plan_tables(const fo_plan *plan, int32_t *tile_of_slot, int32_t *slot_of_tile,
                   int32_t *group_of_slot, int32_t *group_tiles, int64_t *span_off);

/*
 * Consumer work units: unit_off[num_units+1] element bounds (unit u is
 * [unit_off[u], unit_off[u+1])) and group_unit[P+1] (group j owns units
 * [group_unit[j], group_unit[j+1])).  TILE: one unit per group; SUBTILE: R
 * rank segments per group; SUBTOKEN: D destination buckets per group.
 */
int fo_plan_units(const fo_plan *plan, int64_t *unit_off, int32_t *group_unit);

/*
 * Host-side check of the layout the kernels use: off[m * N + n] receives
 * the reordered offset of output element (m, n), computed from the same
 * per-slot records that the device reads.  off has M * N entries.
 */
int fo_plan_offsets(const fo_plan *plan, int64_t *off);

/*
 * Predictive partition search (deep-dive 四、实时调优 › 在线阶段: 预测搜索算法,
 * Algorithm 1).  Scores every composition of the plan's T waves -- 2^(T-1)
 * candidates; the plan's own composition is not used -- with the pages'
 * latency model and returns the best:
 *   compute_end(i) = gemm_seconds / T * (waves of groups 0 .. i)
 *   comm_end(i)    = max(compute_end(i), comm_end(i-1)) + lat(bytes of group i),  comm_end(-1) = 0
 *   prediction     = comm_end(P-1)
 * bytes of a group = its span (elements x 2).  lat() interpolates the
 * sampled curve (curve_bytes[points] > 0, strictly increasing;
 * curve_seconds[points] >= 0) linearly, holds the first sample's latency
 * below it, grows at the last sample's bandwidth beyond it, and is 0 for
 * 0 bytes.  gemm_seconds >= 0 is the whole GEMM's duration.
 * best_comp: host int32[T], receives the winning composition
 *   (*best_num_groups entries); ties keep the first candidate in mask order.
 * all_seconds: NULL or host double[2^(T-1)]: the prediction of candidate
 *   `mask` (bit i set = a group ends after wave i+1) at index mask.
 * Errors: FO_ERR_INVALID for a malformed curve or NULL outputs,
 *   FO_ERR_UNSUPPORTED for T > 24.  Host-only plans are accepted.
 */
int fo_plan_search(const fo_plan *plan, double gemm_seconds, const double *curve_bytes,
                   const double *curve_seconds, int32_t points, int32_t *best_comp,
                   int32_t *best_num_groups, double *best_seconds, double *all_seconds);

/*
 * Signaling GEMM (deep-dive 五 › 扩展主循环 and Epilogue 集成): C = A . B^T
 * with every finished tile stored through the mapping table into
 * `reorder_buf` (M*N elements, the contiguous per-group spans) with
 * stores written through the L2 to the device's point of coherence; once
 * every one of them is complete, one atomic increment of cnt[group], and --
 * by the tile that brings cnt[group] to epoch*|G_group| -- a release store
 * flag[group] = epoch.
 *
 * sig: device uint32[sig_words] (fo_plan_info): the counting table cnt[P] at
 *      word 0 and the flags flag[P] at word flag_offset, the first multiple of
 *      64 words (256 bytes) at or after P, so that with a 256-byte aligned sig
 *      the flags that consumers poll never share a cache line with the
 *      counters every tile increments.  With FO_PLAN_EPOCH_STAMPS the words
 *      from stamp_offset hold one stamp per slot, which the launch sets to
 *      epoch once the slot's tile is stored.  Zero it once before the first epoch.  Epochs start at 1 and increase by 1 per launch on
 *      the same sig, so no reset is needed between launches; after epoch e,
 *      cnt[j] == e*|G_j|.  epoch * max|G_j| must fit in 32 bits.
 * trace: NULL, or device uint64[2*NT + P]: for slot s, trace[2s] = wall
 *      clock at the tile's signal, trace[2s+1] = (workgroup << 32) | the
 *      counter value before the increment; trace[2NT + j] += 1 when group j
 *      fires.  Zero it before the launch.
 */
int fo_gemm_signal(const fo_plan *plan, const void *A, const void *B, void *reorder_buf,
                   uint32_t *sig, uint32_t epoch, uint64_t *trace, hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * launch as fo_gemm_signal, with the signal words (counting table, flags and,
 * for FO_PLAN_EPOCH_STAMPS plans, the stamps) kept in a fixed array of the
 * library's own device memory instead of a caller buffer: 16384 words
 * (64 KiB) per device, held until the process ends.  Plans whose sig_words
 * exceed 16384 are refused with FO_ERR_UNSUPPORTED before anything is
 * enqueued.  No allocation: the array's address is looked up once per device
 * (hipGetSymbolAddress, at the first call on that device).
 *
 * The library chooses the epoch (a counter per device, 1, 2, ...), clears the
 * plan's sig_words words of the array with a small kernel on `stream` ahead
 * of the GEMM (an earlier plan may have left counters where this one keeps
 * its flags), and the GEMM fires each group at |G_j| tiles.  *sig_out receives the array's device
 * address and *epoch_out the epoch: pass both to fo_consume_group or
 * fo_consume_group_gated for this launch's groups.  Every call on a device
 * shares that device's array, which keeps the last call's contents: calls
 * whose GEMMs or consumers overlap on one device race on it, so issue them in
 * order.  A, B and reorder_buf as for fo_gemm_signal.
 */
int fo_gemm_signal_noalloc(const fo_plan *plan, const void *A, const void *B, void *reorder_buf,
                           uint32_t **sig_out, uint32_t *epoch_out, hipStream_t stream);

/*
 * Debug form of fo_gemm_signal that makes the waves physical, so that the
 * counting table's trajectory (deep-dive 一 › 实现方法, the worked example's
 * table after every wave) can be read back: after wave w every workgroup
 * meets at a device-wide barrier, workgroup 0 copies the signal words into
 * snapshots[w*2P ..]: cnt[P] then flag[P], and a second barrier releases
 * wave w+1.  Same arguments and results as fo_gemm_signal otherwise.
 * snapshots: device uint32[T*2P + 2], zeroed by the caller before each
 *      launch; the last two words are the barrier's arrival counter and a
 *      status word, which receives FO_ERR_TIMEOUT if any barrier wait exceeds
 *      2 s (every workgroup then leaves).
 * The launch is cooperative: FO_ERR_UNSUPPORTED if the device cannot hold
 * all W workgroups at once.  For tests and traces, not for the hot path.
 */
int fo_gemm_signal_serialized(const fo_plan *plan, const void *A, const void *B, void *reorder_buf,
                              uint32_t *sig, uint32_t epoch, uint32_t *snapshots, hipStream_t stream);

/*
 * The same GEMM main loop with a plain row-major epilogue and no signaling:
 * C[M, N] row-major.  Reference for the interference check.
 */
int fo_gemm_plain(const fo_plan *plan, const void *A, const void *B, void *C, hipStream_t stream);

/*
 * Consumer: for groups g = g_begin .. g_end-1 in order, wait on the device
 * until flag[g] >= epoch (sig laid out as for fo_gemm_signal), then for every
 * unit of g compute
 *   recv[u] = round(float(send[u]) + float(peer[u]))   (element type, RNE)
 * over the unit's elements (the units of a group tile its span, so the
 * kernel streams the span in one pass).  send, peer, recv are flat M*N buffers in the
 * reordered layout; recv may equal send.  This stands in for the group's
 * collective call on the contiguous span (deep-dive 二 › (1) code box;
 * 五 › 专用监控内核).
 *
 * num_workgroups: persistent grid size, 0 = the device's CU count; at most
 *      the CU count, else FO_ERR_INVALID.  Residency: the consumer's
 *      workgroups wait on the CUs for flags that the GEMM raises, so the GEMM's
 *      W workgroups must still find room beside them.  A GEMM workgroup of the
 *      64x64, 128x128 or 256x128 tile holds up to 384 of a SIMD's 512
 *      registers per lane (two 192-register waves on 256x128) and 144 KiB of
 *      the CU's 160 KiB LDS; a consumer workgroup is one wave per SIMD of at
 *      most 96 registers and no LDS to speak of, so one consumer workgroup per
 *      CU fits beside the GEMM and two do not: a grid above the CU count could
 *      keep GEMM workgroups from being dispatched until the consumer times
 *      out.  A 256x256 workgroup holds 464 registers per lane of every SIMD
 *      (two 232-register waves) and 134 KiB of LDS; with such a plan the
 *      consumer runs in a slim form of at most 48 registers, which fits the
 *      rest.  fo_consume_group_gated uses the same forms.
 * timeout_us: upper bound on any one wait (0 = 2 s).  A workgroup that
 *      waits longer stores FO_ERR_TIMEOUT into *dev_status (if it was still
 *      0) and every workgroup then stops; later spans are left untouched.
 * dev_status: device int32, caller zeroes it; read it after synchronising.
 * trace: NULL, or device uint64[P]: workgroup 0 stores the wall clock at the
 *      moment its wait for group g ended (same clock as fo_gemm_signal's
 *      trace), so a caller can see the consumer start a group while the
 *      GEMM is still running.
 * The GEMM that raises the flags must run on a different stream (see
 * fo_stream_create); the two are linked only through sig.  The consumer
 * occupies few resources so that it can stay resident beside the GEMM.
 */
int fo_consume_group(const fo_plan *plan, const void *send, const void *peer, void *recv,
                     const uint32_t *sig, uint32_t epoch, int32_t g_begin, int32_t g_end,
                     int32_t *dev_status, uint64_t timeout_us, int32_t num_workgroups,
                     uint64_t *trace, hipStream_t stream);

/*
 * Consumer gated by a stream wait instead of a persistent polling grid
 * (deep-dive 五 › 专用监控内核: the signal may reach the transfer stream as an
 * event-like notification rather than through a polling kernel).  For g =
 * g_begin .. g_end-1 in order it enqueues on `stream` a wait until flag[g] >=
 * epoch (hipStreamWaitValue32; the HIP runtime of ROCm 7 carries it out as a
 * one-thread kernel that polls the word, so a single wave waits instead of a
 * workgroup on every CU) and then a streaming kernel over g's span with the
 * same arithmetic as fo_consume_group:
 *   recv[u] = round(float(send[u]) + float(peer[u])).
 * The streaming kernel starts only once the group is signalled, and its grid
 * is sized to the span (several workgroups per CU) instead of being
 * persistent, so nothing of it waits on a CU for the GEMM.
 * The wait has no time limit: the signaling GEMM of `epoch` on the same sig
 * must be enqueued (on another stream) or the stream never proceeds.
 * dev_status: device int32 as for fo_consume_group; receives FO_ERR_STALE
 * from the epoch-stamp check.  trace: NULL, or device uint64[P]: the wall
 * clock when group g's kernel started streaming (workgroup 0), as for
 * fo_consume_group.  FO_ERR_UNSUPPORTED if the device cannot wait on a value
 * (hipDeviceAttributeCanUseStreamWaitValue).  Other arguments and errors as
 * for fo_consume_group.
 */
int fo_consume_group_gated(const fo_plan *plan, const void *send, const void *peer, void *recv,
                           const uint32_t *sig, uint32_t epoch, int32_t g_begin, int32_t g_end,
                           int32_t *dev_status, uint64_t *trace, hipStream_t stream);

/*
 * Post-communication reordering (deep-dive 二、重排机制 › 解决方案: 映射表重排 --
 * the inverse mapping puts each tile back where the GEMM would have stored it;
 * Figure 6 for the three layouts; summary, Figure 5):
 *   out[m*N + n] = reordered[off(m, n)]
 * off() is the plan's layout (fo_plan_offsets).  reordered and out: device,
 * M*N elements, distinct.  Errors: FO_ERR_INVALID for a null or misaligned
 * buffer or a plan without device tables on the current device.
 */
int fo_reorder_post(const fo_plan *plan, const void *reordered, void *out, hipStream_t stream);

/*
 * The same inverse mapping restricted to the tiles of groups g_begin ..
 * g_end-1: only their elements of out are written, the rest of out is left
 * as it is (deep-dive 二 › 解决方案: 映射表重排 -- once a group's
 * communication is done its span holds finished tiles, so they can be put
 * back in place while later groups are still computed or communicated).
 * Calls over a partition of [0, P) write out completely, as fo_reorder_post
 * does.  0 <= g_begin <= g_end <= P, else FO_ERR_INVALID; an empty range
 * enqueues nothing.  Buffers as for fo_reorder_post.
 */
int fo_reorder_post_groups(const fo_plan *plan, int32_t g_begin, int32_t g_end, const void *reordered, void *out,
                           hipStream_t stream);

/*
 * Post-communication reordering fused with the element-wise epilogue
 * (deep-dive 五 › Epilogue 集成: the operations that follow the GEMM -- bias
 * addition, ReLU, SiLU -- run in the reorder's pass, so the output is
 * written once):
 *   out[m*N + n] = round(act(float(reordered[off(m, n)]) + float(bias[e(m)*N + n])))
 * e(m) is the problem (expert) row m belongs to; bias: NULL (no bias) or
 * device, 16-byte aligned, num_problems * N elements of the plan's type.
 * act: fo_act.  One fp32 addition, the activation in fp32, one rounding to
 * nearest even.  reordered and out as for fo_reorder_post.
 */
int fo_reorder_post_ep(const fo_plan *plan, const void *reordered, void *out, const void *bias, int32_t act,
                       hipStream_t stream);

/*
 * Pre-communication reordering as a separate pass (deep-dive 二 › 解决方案: the
 * mapping table gathers the tiles of a group into consecutive addresses so
 * that one collective call can take them; the signaling GEMM does the same in
 * its epilogue):
 *   reordered[off(m, n)] = in[m*N + n]
 * in and reordered: device, M*N elements, distinct.  Errors as for
 * fo_reorder_post.
 */
int fo_reorder_pre(const fo_plan *plan, const void *in, void *reordered, hipStream_t stream);

/*
 * ReduceScatter + AllGather, the first half (deep-dive 二 › 不同通信原语的重排模式,
 * (2) ReduceScatter + AllGather: after the ReduceScatter every rank holds band
 * k of every tile, and these k-th pieces form complete rows).  A SUBTILE plan
 * only (FO_ERR_INVALID otherwise).  Rank k owns the rows whose band inside
 * their tile row is k -- rows m with floor((m mod BM) / (BM/R)) == k, a
 * block-cyclic deal of blocks of BM/R rows -- and keeps them as a row-major
 * shard of M/R rows in increasing row order.  This call writes every rank's
 * shard from its segments of the reordered buffer through the mapping table:
 *   gathered[k*(M/R)*N + i*N + n] = reordered[off(m, n)]
 * for the row m that is the i-th row of rank k.  With the R shards placed back
 * to back, `gathered` is the buffer an AllGather of the shards produces.
 * reordered and gathered: device, M*N elements, distinct.
 */
int fo_reorder_shards(const fo_plan *plan, const void *reordered, void *gathered, hipStream_t stream);

/*
 * ReduceScatter + AllGather, the second half (same passage: the row order
 * after the AllGather is corrected by a local row exchange, a block-cyclic
 * permutation that needs no mapping table and merges with the element-wise
 * operations).  A SUBTILE plan only.  Row m of the output is row
 * k*(M/R) + floor(m / BM)*(BM/R) + (m mod (BM/R)) of `gathered`, with
 * k = floor((m mod BM) / (BM/R)); computed from M, BM and R alone.  With the
 * element-wise epilogue of fo_reorder_post_ep:
 *   out[m*N + n] = round(act(float(gathered[row(m)*N + n]) + float(bias[e(m)*N + n])))
 * bias: NULL or num_problems * N elements; act: fo_act.  gathered and out:
 * device, M*N elements, distinct.  fo_reorder_shards followed by this call
 * gives what fo_reorder_post_ep gives on the same reordered buffer.
 */
int fo_row_exchange(const fo_plan *plan, const void *gathered, void *out, const void *bias, int32_t act,
                    hipStream_t stream);

/*
 * A stream for the GEMM or the consumer side: a HIP stream on the current
 * device with a hardware queue of its own (created with a CU mask that
 * enables every CU, default priority).  Streams that share a hardware queue
 * run their kernels one after another, which would serialise the consumer
 * behind the GEMM instead of running it alongside.  Destroy with
 * fo_stream_destroy.
 */
int fo_stream_create(hipStream_t *out);
int fo_stream_destroy(hipStream_t stream);

/*
 * Measurement aid for the signaling GEMM's roofline, not a step of the method
 * (the pages time their GEMM against its hardware; deep-dive 三 › 调优挑战).
 * Runs nothing but the MFMAs of the GEMM's 256 x 128 tile, v_mfma_f32_16x16x32
 * (dtype: fo_dtype, bf16 or fp16), on operand registers read from `ops`, so
 * its rate is the matrix pipe's ceiling for those values at the clock the
 * part keeps under that load -- without the GEMM's loads, LDS traffic or
 * epilogue.  `workgroups` workgroups of 512 threads (eight waves, two per
 * SIMD); every lane reads 16 vectors of 16 bytes from `ops` (lane i's vectors
 * 16i .. 16i+15, indices modulo ops_bytes / 16: two sets of 4 A operands then
 * 4 B operands), then runs `iters` rounds; a round multiplies, for each set in
 * turn, every (A, B) pair of the set into its own accumulator (A-major, B as
 * the instruction's first operand: 16 MFMAs per set), and the lane stores the
 * sum of its accumulators in out[lane] (fp32, summed in register order).
 *   FLOP per launch = workgroups * 8 * iters * 32 * 2 * 16 * 16 * 32.
 * ops: device, 16-byte aligned, ops_bytes a positive multiple of 16; out:
 * device float[workgroups * 512]; 1 <= workgroups <= 65536; 0 <= iters.
 * FO_ERR_INVALID on any other argument; FO_ERR_HIP if the launch fails.
 */
int fo_mfma_rate(int32_t dtype, const void *ops, int64_t ops_bytes, int32_t workgroups, int32_t iters, float *out,
                 hipStream_t stream);

/* Static description of a status code. */
const char *fo_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* FO_H_ */
