// Enqueue calls of the C ABI: argument checks on the host, then the launchers.
// The enqueue calls allocate nothing, copy nothing from the host and never
// synchronise; only fo_stream_create makes a runtime object (a stream).
#include <cstdint>
#include <vector>

#include "fo_internal.h"

namespace {

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// a plan with device tables, whose device is the current one (its table
// pointers mean nothing on another device)
bool device_ready(const fo_plan *p) {
  if (!p || p->host_only || !p->dev_block) return false;
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev == p->device;
}

// a buffer of M*N elements must be present and 16-byte aligned unless it is empty
bool buf_ok(const fo_plan *p, const void *ptr) { return (p->M * p->N == 0) || (ptr && aligned16(ptr)); }

// operands, reorder buffer, signal words and epoch of a signaling launch on a
// non-empty plan; the counters reach epoch * |G_j|, which must fit in 32 bits
bool signal_args_ok(const fo_plan *p, const void *A, const void *B, const void *reorder_buf, const uint32_t *sig,
                    uint32_t epoch) {
  if (!A || !B || !aligned16(A) || !aligned16(B) || !buf_ok(p, reorder_buf)) return false;
  if (!sig || (reinterpret_cast<uintptr_t>(sig) & 3u) || epoch == 0) return false;
  int32_t max_g = 0;
  for (int32_t v : p->group_tiles) max_g = v > max_g ? v : max_g;
  return (uint64_t)epoch * (uint64_t)max_g <= 0xFFFFFFFFull;
}

}  // namespace

extern "C" {

int fo_gemm_signal(const fo_plan *p, const void *A, const void *B, void *reorder_buf, uint32_t *sig, uint32_t epoch,
                   uint64_t *trace, hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (p->NT == 0) return FO_OK;
  if (!signal_args_ok(p, A, B, reorder_buf, sig, epoch)) return FO_ERR_INVALID;
  if (trace && (reinterpret_cast<uintptr_t>(trace) & 7u)) return FO_ERR_INVALID;
  return fo::launch_gemm(p, A, B, reorder_buf, false, sig, epoch, trace, nullptr, stream);
}

int fo_gemm_signal_serialized(const fo_plan *p, const void *A, const void *B, void *reorder_buf, uint32_t *sig,
                              uint32_t epoch, uint32_t *snapshots, hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (p->NT == 0) return FO_OK;
  if (!signal_args_ok(p, A, B, reorder_buf, sig, epoch)) return FO_ERR_INVALID;
  if (!snapshots || (reinterpret_cast<uintptr_t>(snapshots) & 3u)) return FO_ERR_INVALID;
  return fo::launch_gemm(p, A, B, reorder_buf, false, sig, epoch, nullptr, snapshots, stream);
}

int fo_gemm_plain(const fo_plan *p, const void *A, const void *B, void *C, hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (p->NT == 0) return FO_OK;
  if (!A || !B || !aligned16(A) || !aligned16(B) || !buf_ok(p, C)) return FO_ERR_INVALID;
  return fo::launch_gemm(p, A, B, C, true, nullptr, 0, nullptr, nullptr, stream);
}

int fo_consume_group(const fo_plan *p, const void *send, const void *peer, void *recv, const uint32_t *sig,
                     uint32_t epoch, int32_t g_begin, int32_t g_end, int32_t *dev_status, uint64_t timeout_us,
                     int32_t num_workgroups, uint64_t *trace, hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (g_begin < 0 || g_end > p->P || g_begin > g_end) return FO_ERR_INVALID;
  if (g_begin == g_end) return FO_OK;
  if (!buf_ok(p, send) || !buf_ok(p, peer) || !buf_ok(p, recv)) return FO_ERR_INVALID;
  if (!sig || (reinterpret_cast<uintptr_t>(sig) & 3u) || epoch == 0) return FO_ERR_INVALID;
  if (!dev_status || (reinterpret_cast<uintptr_t>(dev_status) & 3u)) return FO_ERR_INVALID;
  // at most one persistent consumer workgroup per CU, so that the GEMM's workgroups still fit beside them
  if (num_workgroups < 0 || num_workgroups > p->num_cus) return FO_ERR_INVALID;
  const int32_t grid = num_workgroups ? num_workgroups : p->num_cus;
  const uint64_t us = timeout_us ? timeout_us : 2000000ull;
  if (us > (1ull << 40)) return FO_ERR_INVALID;
  if (trace && (reinterpret_cast<uintptr_t>(trace) & 7u)) return FO_ERR_INVALID;
  return fo::launch_consume(p, send, peer, recv, sig, epoch, g_begin, g_end, dev_status, us * p->ticks_per_us, grid,
                            trace, stream);
}

int fo_consume_group_gated(const fo_plan *p, const void *send, const void *peer, void *recv, const uint32_t *sig,
                           uint32_t epoch, int32_t g_begin, int32_t g_end, int32_t *dev_status, uint64_t *trace,
                           hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (g_begin < 0 || g_end > p->P || g_begin > g_end) return FO_ERR_INVALID;
  if (g_begin == g_end) return FO_OK;
  if (!buf_ok(p, send) || !buf_ok(p, peer) || !buf_ok(p, recv)) return FO_ERR_INVALID;
  if (!sig || (reinterpret_cast<uintptr_t>(sig) & 3u) || epoch == 0) return FO_ERR_INVALID;
  if (!dev_status || (reinterpret_cast<uintptr_t>(dev_status) & 3u)) return FO_ERR_INVALID;
  if (trace && (reinterpret_cast<uintptr_t>(trace) & 7u)) return FO_ERR_INVALID;
  if (!p->can_wait_value) return FO_ERR_UNSUPPORTED;
  const uint32_t *flag = sig + p->flag_offset();
  for (int32_t g = g_begin; g < g_end; ++g) {
    // the stream proceeds once flag[g] >= epoch (a stream wait), then runs the group's kernel
    if (hipStreamWaitValue32(stream, const_cast<uint32_t *>(flag + g), epoch, hipStreamWaitValueGte, 0xFFFFFFFFu) !=
        hipSuccess)
      return FO_ERR_HIP;
    const int rc = fo::launch_consume_ready(p, send, peer, recv, sig, epoch, g, dev_status, trace, stream);
    if (rc != FO_OK) return rc;
  }
  return FO_OK;
}

int fo_reorder_shards(const fo_plan *p, const void *reordered, void *gathered, hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (p->mode != FO_MODE_SUBTILE) return FO_ERR_INVALID;
  if (!buf_ok(p, reordered) || !buf_ok(p, gathered)) return FO_ERR_INVALID;
  return fo::launch_shards(p, reordered, gathered, stream);
}

int fo_row_exchange(const fo_plan *p, const void *gathered, void *out, const void *bias, int32_t act,
                    hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (p->mode != FO_MODE_SUBTILE) return FO_ERR_INVALID;
  if (!buf_ok(p, gathered) || !buf_ok(p, out)) return FO_ERR_INVALID;
  if (bias && !aligned16(bias)) return FO_ERR_INVALID;
  if (act != FO_ACT_NONE && act != FO_ACT_RELU && act != FO_ACT_SILU) return FO_ERR_INVALID;
  return fo::launch_row_exchange(p, gathered, out, bias, act, stream);
}

int fo_reorder_post(const fo_plan *p, const void *reordered, void *out, hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (!buf_ok(p, reordered) || !buf_ok(p, out)) return FO_ERR_INVALID;
  return fo::launch_reorder(p, reordered, out, true, 0, p->NT, stream);
}

int fo_reorder_post_groups(const fo_plan *p, int32_t g_begin, int32_t g_end, const void *reordered, void *out,
                           hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (g_begin < 0 || g_end > p->P || g_begin > g_end) return FO_ERR_INVALID;
  if (!buf_ok(p, reordered) || !buf_ok(p, out)) return FO_ERR_INVALID;
  int32_t first = 0, last = 0;  // slots of groups [g_begin, g_end): consecutive, in group order
  for (int32_t g = 0; g < g_end; ++g) {
    if (g < g_begin) first += p->group_tiles[g];
    last += p->group_tiles[g];
  }
  return fo::launch_reorder(p, reordered, out, true, first, last, stream);
}

int fo_reorder_post_ep(const fo_plan *p, const void *reordered, void *out, const void *bias, int32_t act,
                       hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (!buf_ok(p, reordered) || !buf_ok(p, out)) return FO_ERR_INVALID;
  if (bias && !aligned16(bias)) return FO_ERR_INVALID;
  if (act != FO_ACT_NONE && act != FO_ACT_RELU && act != FO_ACT_SILU) return FO_ERR_INVALID;
  return fo::launch_post_ep(p, reordered, out, bias, act, stream);
}

int fo_reorder_pre(const fo_plan *p, const void *in, void *reordered, hipStream_t stream) {
  if (!device_ready(p)) return FO_ERR_INVALID;
  if (!buf_ok(p, in) || !buf_ok(p, reordered)) return FO_ERR_INVALID;
  return fo::launch_reorder(p, in, reordered, false, 0, p->NT, stream);
}

int fo_mfma_rate(int32_t dtype, const void *ops, int64_t ops_bytes, int32_t workgroups, int32_t iters, float *out,
                 hipStream_t stream) {
  if (dtype != FO_BF16 && dtype != FO_FP16) return FO_ERR_INVALID;
  if (!ops || !aligned16(ops) || ops_bytes < 16 || ops_bytes % 16 != 0) return FO_ERR_INVALID;
  if (workgroups < 1 || workgroups > 65536 || iters < 0) return FO_ERR_INVALID;
  if (!out || (reinterpret_cast<uintptr_t>(out) & 3u)) return FO_ERR_INVALID;
  return fo::launch_mfma_rate(dtype, ops, ops_bytes, workgroups, iters, out, stream);
}

int fo_stream_create(hipStream_t *out) {
  if (!out) return FO_ERR_INVALID;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return FO_ERR_HIP;
  // every CU enabled; a masked stream is given a hardware queue of its own
  std::vector<uint32_t> mask((cus + 31) / 32, 0xFFFFFFFFu);
  if (cus % 32) mask.back() = (1u << (cus % 32)) - 1u;
  hipStream_t s = nullptr;
  if (hipExtStreamCreateWithCUMask(&s, (uint32_t)mask.size(), mask.data()) != hipSuccess) return FO_ERR_HIP;
  *out = s;
  return FO_OK;
}

int fo_stream_destroy(hipStream_t stream) {
  if (!stream) return FO_ERR_INVALID;
  return hipStreamDestroy(stream) == hipSuccess ? FO_OK : FO_ERR_HIP;
}

}  // extern "C"
