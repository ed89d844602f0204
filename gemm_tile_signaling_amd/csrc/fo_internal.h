// Internal declarations shared by the planner and the HIP kernels of libfo.
//
// The planner (plan.cpp) turns a fo_plan_desc into per-slot records and a few
// small tables; the kernels read only those.  The row-offset function below
// is the single definition of the reordered layout used by the GEMM
// epilogue, both reorder kernels and the host-side fo_plan_offsets check.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/fo.h"

namespace fo {

// Layout of the destination written by a GEMM epilogue or read by a reorder.
enum LayoutMode : int32_t {
  kRowMajor = 0,   // C[m, n] at m * N + n
  kBanded = 1,     // TILE (one band of BM rows) and SUBTILE (R bands per tile)
  kSubtoken = 2,   // SUBTOKEN: each tile row lands in its destination's bucket
};

// One record per slot (= dispatch index b).  40 bytes.
struct TileDesc {
  int32_t row0;        // first output row of the tile (rows of all problems stacked)
  int32_t col0;        // first output column
  int32_t rows;        // valid rows (< BM only for the last tile row of a problem)
  int32_t cols;        // valid columns (< BN only at the right edge)
  int32_t problem;     // which B matrix (expert) the tile multiplies with
  int32_t group;       // wave group j
  int64_t base;        // kBanded: reordered offset of the tile's first row
  int64_t band_stride; // kBanded: distance between consecutive row bands
};
static_assert(sizeof(TileDesc) == 40, "TileDesc layout");

struct Layout {
  int32_t mode;            // LayoutMode
  int32_t band_rows;       // kBanded: rows per band (BM for TILE, BM / R for SUBTILE)
  int32_t D;               // kSubtoken: number of destination buckets
  int32_t pad_;
  int64_t N;               // kRowMajor: row length of C
  const int64_t *dbase;    // kSubtoken: [NT * D] offset of slot s's first row bound for d
  const int32_t *row_dest; // kSubtoken: [M] destination of each output row
  const int32_t *row_rank; // kSubtoken: [M] rank of the row among its tile row's rows with the same destination
};

// Reordered offset of the first element of row r of the tile at `slot`.
// Element (r, c) of the tile is at row_offset(...) + c.
__host__ __device__ inline int64_t row_offset(const Layout &L, const TileDesc &t, int32_t slot, int32_t r) {
  if (L.mode == kRowMajor) return (int64_t)(t.row0 + r) * L.N + t.col0;
  if (L.mode == kBanded) {
    const int32_t k = r / L.band_rows, rr = r - k * L.band_rows;
    return t.base + (int64_t)k * t.band_stride + (int64_t)rr * t.cols;
  }
  const int32_t m = t.row0 + r;
  return L.dbase[(int64_t)slot * L.D + L.row_dest[m]] + (int64_t)L.row_rank[m] * t.cols;
}

}  // namespace fo

// The opaque plan behind the C ABI.
struct fo_plan {
  fo_plan_desc desc{};           // copy; host pointers in it are not kept
  int64_t M = 0, N = 0, K = 0;
  int32_t BM = 0, BN = 0, S = 0, W = 0;
  int32_t NT = 0, T = 0, P = 0;
  int32_t mode = 0, ranks = 1, dtype = 0, num_problems = 1;
  int32_t band_rows = 0;
  int32_t min_tile_rows = 0, min_tile_cols = 0;  // smallest extent of any tile (ragged edges)
  uint32_t flags = 0;             // FO_PLAN_* bits
  bool host_only = false;
  bool can_wait_value = false;    // the device's queues can wait on a memory value
  int32_t device = -1;
  int32_t num_cus = 0;
  uint64_t ticks_per_us = 100;   // device wall clock rate

  std::vector<int64_t> m_per_problem;
  std::vector<int32_t> tile_of_slot, slot_of_tile, group_of_slot, group_tiles;
  std::vector<int64_t> span_off;         // P + 1
  std::vector<int64_t> unit_off;         // units + 1
  std::vector<int32_t> group_unit;       // P + 1
  std::vector<fo::TileDesc> slots;       // NT
  std::vector<int64_t> dbase;            // NT * D (subtoken)
  std::vector<int32_t> row_dest, row_rank;  // M (subtoken)
  std::vector<int32_t> group_first;      // P + 1: first slot of each group
  std::vector<int32_t> problem_row0;     // num_problems + 1: first output row of each problem

  // device copies (one allocation)
  void *dev_block = nullptr;
  const fo::TileDesc *d_slots = nullptr;
  const int32_t *d_group_tiles = nullptr;
  const int64_t *d_unit_off = nullptr;
  const int32_t *d_group_unit = nullptr;
  const int64_t *d_dbase = nullptr;
  const int32_t *d_row_dest = nullptr;
  const int32_t *d_row_rank = nullptr;
  const int32_t *d_group_first = nullptr;
  const int32_t *d_problem_row0 = nullptr;

  // Signal words: cnt[P] at word 0, flag[P] from the next multiple of 64 words,
  // so the lines consumers poll are not the lines every tile's atomic updates.
  // With FO_PLAN_EPOCH_STAMPS, one stamp word per slot follows, from the next
  // multiple of 64 words after the flags.
  int32_t flag_offset() const { return (P + 63) / 64 * 64; }
  bool stamps() const { return (flags & FO_PLAN_EPOCH_STAMPS) != 0; }
  int32_t stamp_offset() const { return stamps() ? flag_offset() + (P + 63) / 64 * 64 : -1; }
  int32_t sig_words() const { return stamps() ? stamp_offset() + NT : flag_offset() + P; }

  fo::Layout layout(bool device_side) const {
    fo::Layout L{};
    L.mode = mode == FO_MODE_SUBTOKEN ? fo::kSubtoken : fo::kBanded;
    L.band_rows = band_rows;
    L.D = mode == FO_MODE_SUBTOKEN ? ranks : 1;
    L.N = N;
    L.dbase = device_side ? d_dbase : dbase.data();
    L.row_dest = device_side ? d_row_dest : row_dest.data();
    L.row_rank = device_side ? d_row_rank : row_rank.data();
    return L;
  }
};

namespace fo {

// Kernel launchers (the .hip files).  Arguments are validated by the caller.
// counts_cleared: the counting table was zeroed for this launch, so a group fires at |G_g|
// instead of epoch * |G_g| (the signal words are otherwise monotonic across epochs)
int launch_gemm(const fo_plan *p, const void *A, const void *B, void *C, bool rowmajor,
                uint32_t *sig, uint32_t epoch, uint64_t *trace, uint32_t *serial, hipStream_t s,
                bool counts_cleared = false);
int launch_consume(const fo_plan *p, const void *send, const void *peer, void *recv,
                   const uint32_t *sig, uint32_t epoch, int32_t g_begin, int32_t g_end,
                   int32_t *status, uint64_t timeout_ticks, int32_t grid, uint64_t *trace, hipStream_t s);
// one group, launched after its signal: no polling, a grid sized to the span
int launch_consume_ready(const fo_plan *p, const void *send, const void *peer, void *recv, const uint32_t *sig,
                         uint32_t epoch, int32_t g, int32_t *status, uint64_t *trace, hipStream_t s);
int launch_shards(const fo_plan *p, const void *src, void *gathered, hipStream_t s);
int launch_row_exchange(const fo_plan *p, const void *gathered, void *out, const void *bias, int act,
                        hipStream_t s);
int launch_reorder(const fo_plan *p, const void *src, void *dst, bool to_rowmajor, int32_t slot_begin,
                   int32_t slot_end, hipStream_t s);
int launch_post_ep(const fo_plan *p, const void *src, void *dst, const void *bias, int act, hipStream_t s);
int launch_mfma_rate(int dtype, const void *ops, int64_t ops_bytes, int32_t workgroups, int32_t iters, float *out,
                     hipStream_t s);

}  // namespace fo
