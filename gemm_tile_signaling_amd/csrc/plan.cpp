// Wave-group planner: tile grid, swizzled dispatch order, waves, groups,
// mapping table, thresholds, spans, consumer units and the per-slot records
// the kernels read.
//
// Method: deep-dive page "FlashOverlap: 信号驱动计算通信重叠论文详解",
//   一、信号机制 (waves, block swizzling, wave groups, group-level tile counting),
//   二、重排机制 (mapping table; reorder patterns for AllReduce, ReduceScatter
//   and All-to-All, Figure 6), 三、Wave Group 划分设计空间 (partitions of T).
// Readings for what the pages leave open are stated in fo.h next to the
// fields they govern.
#include <algorithm>
#include <cstring>
#include <new>

#include "fo_internal.h"

namespace {

bool valid_tile(int32_t BM, int32_t BN) {
  return (BM == 256 && BN == 256) || (BM == 256 && BN == 128) || (BM == 128 && BN == 128) || (BM == 64 && BN == 64);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Grouped-M order of width S over a tm_n x tn_n grid: dispatch index b ->
// row-major tile index.  Bands of S tile rows (the last one h <= S rows),
// walked column by column, each column top to bottom.
void swizzle(int32_t tm_n, int32_t tn_n, int32_t S, int32_t first, std::vector<int32_t> &out) {
  const int64_t per_band = (int64_t)S * tn_n;
  for (int64_t b = 0; b < (int64_t)tm_n * tn_n; ++b) {
    const int64_t band = b / per_band, loc = b % per_band;
    const int64_t h = std::min<int64_t>(S, tm_n - band * S);
    const int64_t tm = band * S + loc % h, tn = loc / h;
    out.push_back(first + (int32_t)(tm * tn_n + tn));
  }
}

int upload(fo_plan *p) {
  // one device block: slots, group_tiles, unit_off, group_unit, dbase, row_dest, row_rank,
  // group_first, problem_row0
  constexpr int kTables = 9;
  auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t n_slots = p->slots.size() * sizeof(fo::TileDesc);
  const size_t n_gt = p->group_tiles.size() * sizeof(int32_t);
  const size_t n_uo = p->unit_off.size() * sizeof(int64_t);
  const size_t n_gu = p->group_unit.size() * sizeof(int32_t);
  const size_t n_db = p->dbase.size() * sizeof(int64_t);
  const size_t n_rd = p->row_dest.size() * sizeof(int32_t);
  const size_t n_rr = p->row_rank.size() * sizeof(int32_t);
  const size_t n_gf = p->group_first.size() * sizeof(int32_t);
  const size_t n_pr = p->problem_row0.size() * sizeof(int32_t);
  size_t off[kTables];
  size_t total = 0;
  const size_t sizes[kTables] = {n_slots, n_gt, n_uo, n_gu, n_db, n_rd, n_rr, n_gf, n_pr};
  for (int i = 0; i < kTables; ++i) { off[i] = total; total += align(sizes[i] ? sizes[i] : 1); }
  if (hipGetDevice(&p->device) != hipSuccess) return FO_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, p->device) != hipSuccess) return FO_ERR_HIP;
  if (!fo_arch_supported(prop.gcnArchName)) return FO_ERR_UNSUPPORTED;
  int cus = 0, clk_khz = 0, wait_value = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device) != hipSuccess) return FO_ERR_HIP;
  if (hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeWallClockRate, p->device) != hipSuccess) return FO_ERR_HIP;
  if (hipDeviceGetAttribute(&wait_value, hipDeviceAttributeCanUseStreamWaitValue, p->device) != hipSuccess)
    wait_value = 0;
  p->can_wait_value = wait_value != 0;
  p->num_cus = cus;
  p->ticks_per_us = clk_khz > 0 ? (uint64_t)clk_khz / 1000u : 100u;
  if (p->ticks_per_us == 0) p->ticks_per_us = 1;
  void *blk = nullptr;
  if (hipMalloc(&blk, total) != hipSuccess) return FO_ERR_NOMEM;
  p->dev_block = blk;
  char *base = static_cast<char *>(blk);
  const void *src[kTables] = {p->slots.data(),    p->group_tiles.data(), p->unit_off.data(),
                              p->group_unit.data(), p->dbase.data(),   p->row_dest.data(),
                              p->row_rank.data(),   p->group_first.data(), p->problem_row0.data()};
  for (int i = 0; i < kTables; ++i)
    if (sizes[i] && hipMemcpy(base + off[i], src[i], sizes[i], hipMemcpyHostToDevice) != hipSuccess)
      return FO_ERR_HIP;
  p->d_slots = reinterpret_cast<const fo::TileDesc *>(base + off[0]);
  p->d_group_tiles = reinterpret_cast<const int32_t *>(base + off[1]);
  p->d_unit_off = reinterpret_cast<const int64_t *>(base + off[2]);
  p->d_group_unit = reinterpret_cast<const int32_t *>(base + off[3]);
  p->d_dbase = n_db ? reinterpret_cast<const int64_t *>(base + off[4]) : nullptr;
  p->d_row_dest = n_rd ? reinterpret_cast<const int32_t *>(base + off[5]) : nullptr;
  p->d_row_rank = n_rr ? reinterpret_cast<const int32_t *>(base + off[6]) : nullptr;
  p->d_group_first = reinterpret_cast<const int32_t *>(base + off[7]);
  p->d_problem_row0 = reinterpret_cast<const int32_t *>(base + off[8]);
  return FO_OK;
}

int build(const fo_plan_desc *d, fo_plan *p) {
  if (d->num_problems < 1 || !d->m_per_problem) return FO_ERR_INVALID;
  if (d->N <= 0 || d->K <= 0 || d->N % 8 != 0) return FO_ERR_INVALID;
  if (d->N > INT32_MAX || d->K > INT32_MAX) return FO_ERR_INVALID;
  if (d->K % 64 != 0) return FO_ERR_UNSUPPORTED;
  if (d->dtype != FO_BF16 && d->dtype != FO_FP16) return FO_ERR_UNSUPPORTED;
  if (d->b_layout == FO_B_KN) return FO_ERR_UNSUPPORTED;
  if (d->b_layout != FO_B_NK) return FO_ERR_INVALID;
  if (d->mode < FO_MODE_TILE || d->mode > FO_MODE_SUBTOKEN) return FO_ERR_INVALID;
  if (d->flags & ~(FO_PLAN_HOST_ONLY | FO_PLAN_EPOCH_STAMPS)) return FO_ERR_INVALID;
  p->desc = *d;
  p->flags = d->flags;
  p->host_only = (d->flags & FO_PLAN_HOST_ONLY) != 0;
  p->N = d->N;
  p->K = d->K;
  p->BM = d->BM ? d->BM : 256;
  p->BN = d->BN ? d->BN : 128;
  if ((d->BM == 0) != (d->BN == 0) || !valid_tile(p->BM, p->BN)) return FO_ERR_UNSUPPORTED;
  // The GEMM addresses a tile's A and B rows with 32-bit byte offsets from the
  // tile's first row: every offset stays below max(BM, BN) * K * 2.
  if ((int64_t)std::max(p->BM, p->BN) * p->K * 2 > (int64_t)UINT32_MAX) return FO_ERR_UNSUPPORTED;
  p->S = d->swizzle ? d->swizzle : 4;
  if (p->S < 1) return FO_ERR_INVALID;
  p->mode = d->mode;
  p->ranks = d->ranks;
  p->dtype = d->dtype;
  p->num_problems = d->num_problems;
  if (d->mode == FO_MODE_TILE) p->ranks = 1;
  if (p->ranks < 1 || p->ranks > 1024) return FO_ERR_INVALID;

  int64_t M = 0;
  p->m_per_problem.assign(d->m_per_problem, d->m_per_problem + d->num_problems);
  for (int64_t m : p->m_per_problem) {
    if (m < 0) return FO_ERR_INVALID;
    M += m;
  }
  if (M > INT32_MAX) return FO_ERR_INVALID;
  // The consumer and the reorders address each buffer with 32-bit byte offsets:
  // at most 2^30 elements (2 GiB) keeps every offset they form, including the
  // ones a thread computes past the end of a unit, below 2^32.
  if (M * p->N > (int64_t(1) << 30)) return FO_ERR_UNSUPPORTED;
  p->M = M;

  if (p->mode == FO_MODE_SUBTILE) {
    if (p->BM % p->ranks != 0 || p->N % p->BN != 0) return FO_ERR_INVALID;
    for (int64_t m : p->m_per_problem)
      if (m % p->BM != 0) return FO_ERR_INVALID;
  }
  if (p->mode == FO_MODE_SUBTOKEN && M > 0) {
    if (!d->row_dest) return FO_ERR_INVALID;
    p->row_dest.assign(d->row_dest, d->row_dest + M);
    for (int32_t v : p->row_dest)
      if (v < 0 || v >= p->ranks) return FO_ERR_INVALID;
  }

  // tile grid (row-major per problem, problems concatenated) and dispatch order
  const int32_t tn_n = (int32_t)cdiv(p->N, p->BN);
  std::vector<fo::TileDesc> tiles;
  int64_t row_base = 0;
  for (int32_t e = 0; e < p->num_problems; ++e) {
    const int64_t m = p->m_per_problem[e];
    const int32_t tm_n = (int32_t)cdiv(m, p->BM);
    const int32_t first = (int32_t)tiles.size();
    for (int32_t tm = 0; tm < tm_n; ++tm)
      for (int32_t tn = 0; tn < tn_n; ++tn) {
        fo::TileDesc t{};
        t.row0 = (int32_t)(row_base + (int64_t)tm * p->BM);
        t.col0 = tn * p->BN;
        t.rows = (int32_t)std::min<int64_t>(p->BM, m - (int64_t)tm * p->BM);
        t.cols = (int32_t)std::min<int64_t>(p->BN, p->N - (int64_t)tn * p->BN);
        t.problem = e;
        tiles.push_back(t);
      }
    if (tm_n) swizzle(tm_n, tn_n, p->S, first, p->tile_of_slot);
    row_base += m;
  }
  if (tiles.size() > (size_t)INT32_MAX / 2) return FO_ERR_INVALID;
  p->NT = (int32_t)tiles.size();
  if (d->dispatch_order) {
    std::vector<char> seen(p->NT, 0);
    for (int32_t b = 0; b < p->NT; ++b) {
      const int32_t t = d->dispatch_order[b];
      if (t < 0 || t >= p->NT || seen[t]) return FO_ERR_INVALID;
      seen[t] = 1;
      p->tile_of_slot[b] = t;
    }
  }
  p->slot_of_tile.assign(p->NT, 0);
  for (int32_t s = 0; s < p->NT; ++s) p->slot_of_tile[p->tile_of_slot[s]] = s;

  // waves and groups
  if (d->wave_size < 0) return FO_ERR_INVALID;
  p->W = d->wave_size;
  if (p->W == 0) {
    if (p->host_only) {
      p->W = 256;
    } else {
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return FO_ERR_HIP;
      p->W = cus;
    }
  }
  p->T = p->NT ? (int32_t)cdiv(p->NT, p->W) : 0;
  std::vector<int32_t> comp;
  if (d->num_groups == 0) {
    comp.assign(p->T, 1);
  } else {
    if (d->num_groups < 0 || !d->waves_per_group) return FO_ERR_INVALID;
    int64_t sum = 0;
    for (int32_t j = 0; j < d->num_groups; ++j) {
      if (d->waves_per_group[j] < 1) return FO_ERR_INVALID;
      sum += d->waves_per_group[j];
      comp.push_back(d->waves_per_group[j]);
    }
    if (sum != p->T) return FO_ERR_INVALID;
  }
  p->P = (int32_t)comp.size();
  std::vector<int32_t> group_of_wave;
  for (int32_t j = 0; j < p->P; ++j) group_of_wave.insert(group_of_wave.end(), comp[j], j);
  p->group_of_slot.resize(p->NT);
  p->group_tiles.assign(p->P, 0);
  for (int32_t s = 0; s < p->NT; ++s) {
    const int32_t g = group_of_wave[s / p->W];
    p->group_of_slot[s] = g;
    p->group_tiles[g] += 1;
  }
  std::vector<int32_t> first_slot(p->P + 1, p->NT);
  for (int32_t s = p->NT - 1; s >= 0; --s) first_slot[p->group_of_slot[s]] = s;
  p->group_first = first_slot;
  p->problem_row0.assign(1, 0);
  for (int64_t m : p->m_per_problem) p->problem_row0.push_back(p->problem_row0.back() + (int32_t)m);

  // per-slot records and spans
  p->slots.resize(p->NT);
  for (int32_t s = 0; s < p->NT; ++s) {
    p->slots[s] = tiles[p->tile_of_slot[s]];
    p->slots[s].group = p->group_of_slot[s];
  }
  p->min_tile_rows = p->BM;
  p->min_tile_cols = p->BN;
  for (const fo::TileDesc &t : p->slots) {
    p->min_tile_rows = std::min(p->min_tile_rows, t.rows);
    p->min_tile_cols = std::min(p->min_tile_cols, t.cols);
  }
  p->span_off.assign(p->P + 1, 0);
  for (int32_t s = 0; s < p->NT; ++s)
    p->span_off[p->group_of_slot[s] + 1] += (int64_t)p->slots[s].rows * p->slots[s].cols;
  for (int32_t j = 0; j < p->P; ++j) p->span_off[j + 1] += p->span_off[j];

  p->unit_off.clear();
  p->group_unit.assign(1, 0);
  if (p->mode == FO_MODE_TILE) {
    p->band_rows = p->BM;
    int64_t pos = 0;
    for (int32_t s = 0; s < p->NT; ++s) {
      p->slots[s].base = pos;
      p->slots[s].band_stride = 0;
      pos += (int64_t)p->slots[s].rows * p->slots[s].cols;
    }
    for (int32_t j = 0; j < p->P; ++j) {
      p->unit_off.push_back(p->span_off[j]);
      p->group_unit.push_back(j + 1);
    }
  } else if (p->mode == FO_MODE_SUBTILE) {
    p->band_rows = p->BM / p->ranks;
    const int64_t q = (int64_t)p->band_rows * p->BN;
    for (int32_t s = 0; s < p->NT; ++s) {
      const int32_t j = p->group_of_slot[s];
      const int64_t n_j = p->group_tiles[j];
      p->slots[s].base = p->span_off[j] + (int64_t)(s - first_slot[j]) * q;
      p->slots[s].band_stride = n_j * q;
    }
    for (int32_t j = 0; j < p->P; ++j) {
      for (int32_t k = 0; k < p->ranks; ++k)
        p->unit_off.push_back(p->span_off[j] + (int64_t)k * p->group_tiles[j] * q);
      p->group_unit.push_back((j + 1) * p->ranks);
    }
  } else {  // SUBTOKEN
    p->band_rows = p->BM;
    const int32_t D = p->ranks;
    p->row_rank.assign(M, 0);
    // rank of each row among the rows of its tile row with the same destination
    std::vector<int32_t> seen(D);
    for (const fo::TileDesc &t : tiles) {
      if (t.col0 != 0) continue;  // one pass per tile row
      std::fill(seen.begin(), seen.end(), 0);
      for (int32_t r = 0; r < t.rows; ++r) {
        const int32_t m = t.row0 + r;
        p->row_rank[m] = seen[p->row_dest[m]]++;
      }
    }
    p->dbase.assign((size_t)p->NT * D, 0);
    for (int32_t j = 0; j < p->P; ++j) {
      int64_t pos = p->span_off[j];
      for (int32_t dd = 0; dd < D; ++dd) {
        p->unit_off.push_back(pos);
        for (int32_t s = first_slot[j]; s < p->NT && p->group_of_slot[s] == j; ++s) {
          const fo::TileDesc &t = p->slots[s];
          p->dbase[(size_t)s * D + dd] = pos;
          int64_t n = 0;
          for (int32_t r = 0; r < t.rows; ++r) n += p->row_dest[t.row0 + r] == dd;
          pos += n * t.cols;
        }
      }
      p->group_unit.push_back((j + 1) * D);
    }
  }
  p->unit_off.push_back(p->P ? p->span_off[p->P] : 0);
  if (p->unit_off.size() == 1) p->unit_off[0] = 0;

  if (!p->host_only) return upload(p);
  return FO_OK;
}

}  // namespace

extern "C" {

int fo_plan_groups(const fo_plan_desc *desc, fo_plan **out) {
  if (!desc || !out) return FO_ERR_INVALID;
  fo_plan *p = new (std::nothrow) fo_plan();
  if (!p) return FO_ERR_NOMEM;
  int rc;
  try {
    rc = build(desc, p);
  } catch (const std::bad_alloc &) {
    rc = FO_ERR_NOMEM;
  } catch (...) {
    rc = FO_ERR_INVALID;
  }
  if (rc != FO_OK) {
    fo_plan_destroy(p);
    return rc;
  }
  *out = p;
  return FO_OK;
}

int fo_plan_destroy(fo_plan *p) {
  if (!p) return FO_ERR_INVALID;
  int rc = FO_OK;
  if (p->dev_block && hipFree(p->dev_block) != hipSuccess) rc = FO_ERR_HIP;
  delete p;
  return rc;
}

int fo_plan_info_get(const fo_plan *p, fo_plan_info *o) {
  if (!p || !o) return FO_ERR_INVALID;
  o->M = p->M;
  o->N = p->N;
  o->K = p->K;
  o->BM = p->BM;
  o->BN = p->BN;
  o->swizzle = p->S;
  o->wave_size = p->W;
  o->NT = p->NT;
  o->T = p->T;
  o->P = p->P;
  o->num_units = (int32_t)p->unit_off.size() - 1;
  o->mode = p->mode;
  o->ranks = p->ranks;
  o->dtype = p->dtype;
  o->num_problems = p->num_problems;
  o->device = p->host_only ? -1 : p->device;
  o->clock_khz = p->host_only ? 0 : (int32_t)(p->ticks_per_us * 1000u);
  o->sig_words = p->sig_words();
  o->flag_offset = p->flag_offset();
  o->stamp_offset = p->stamp_offset();
  o->flags = (int32_t)p->flags;
  return FO_OK;
}

int fo_arch_supported(const char *arch) {
  if (!arch) return 0;
  // the processor name ends at the first ':' (target features follow)
  const char *want = "gfx950";
  size_t i = 0;
  for (; want[i]; ++i)
    if (arch[i] != want[i]) return 0;
  return arch[i] == '\0' || arch[i] == ':';
}

int fo_plan_tables(const fo_plan *p, int32_t *tile_of_slot, int32_t *slot_of_tile, int32_t *group_of_slot,
                   int32_t *group_tiles, int64_t *span_off) {
  if (!p) return FO_ERR_INVALID;
  auto cp = [](auto *dst, const auto &v) {
    if (dst && !v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(v[0]));
  };
  cp(tile_of_slot, p->tile_of_slot);
  cp(slot_of_tile, p->slot_of_tile);
  cp(group_of_slot, p->group_of_slot);
  cp(group_tiles, p->group_tiles);
  cp(span_off, p->span_off);
  return FO_OK;
}

int fo_plan_units(const fo_plan *p, int64_t *unit_off, int32_t *group_unit) {
  if (!p) return FO_ERR_INVALID;
  if (unit_off) std::memcpy(unit_off, p->unit_off.data(), p->unit_off.size() * sizeof(int64_t));
  if (group_unit) std::memcpy(group_unit, p->group_unit.data(), p->group_unit.size() * sizeof(int32_t));
  return FO_OK;
}

int fo_plan_offsets(const fo_plan *p, int64_t *off) {
  if (!p || (!off && p->M * p->N > 0)) return FO_ERR_INVALID;
  const fo::Layout L = p->layout(false);
  for (int32_t s = 0; s < p->NT; ++s) {
    const fo::TileDesc &t = p->slots[s];
    for (int32_t r = 0; r < t.rows; ++r) {
      const int64_t ro = fo::row_offset(L, t, s, r);
      int64_t *dst = off + (int64_t)(t.row0 + r) * p->N + t.col0;
      for (int32_t c = 0; c < t.cols; ++c) dst[c] = ro + c;
    }
  }
  return FO_OK;
}

const char *fo_status_string(int code) {
  switch (code) {
    case FO_OK: return "ok";
    case FO_ERR_INVALID: return "invalid argument";
    case FO_ERR_UNSUPPORTED: return "unsupported configuration";
    case FO_ERR_HIP: return "HIP runtime error";
    case FO_ERR_NOMEM: return "out of memory";
    case FO_ERR_TIMEOUT: return "consumer wait timed out";
    case FO_ERR_STALE: return "consumer read a tile stamp of an older epoch after the signal";
    default: return "unknown status";
  }
}

}  // extern "C"
