// The signaling GEMM for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): fo_gemm_signal with its signal words -- the counting table,
// the flags and the optional epoch stamps, which fo_gemm_signal takes as a
// caller buffer -- kept in a fixed array of the library's own device memory.
//
// The array is a file-scope __device__ variable of kStaticSigWords words.
// Its device address is looked up once per device with hipGetSymbolAddress
// (the variable's name on the host is only a stand-in and must never be
// passed to a kernel) and kept per device.  Every call on one device shares
// that device's array, so:
//   * the library hands out the epochs (one counter per device, 1, 2, ...),
//     so a flag left by an earlier call is always older than the current
//     epoch, whatever plan raised it;
//   * the plan's signal words, [0, sig_words), are cleared for each call by a
//     small fill kernel on the caller's stream ahead of the GEMM: a previous
//     plan with another layout may have left its counters where this plan
//     keeps its flags (a counter at or above the new epoch would release the
//     consumer early) or its flags where this plan counts; the GEMM then
//     fires a group at |G_j| instead of epoch * |G_j|;
//   * calls whose GEMMs or consumers overlap on one device race on the array:
//     a caller issues them in order (one stream, or ordered streams).
#include <mutex>

#include "../fo_internal.h"

namespace {

constexpr int32_t kStaticSigWords = 16384;  // 64 KiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint32_t scratch[kStaticSigWords];

std::mutex g_mu;
uint32_t *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up
uint32_t g_epoch[kMaxDevices];     // last epoch handed out on each device

__global__ void clear_words(uint32_t *w, int32_t n) {
  for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) w[i] = 0u;
}

}  // namespace

extern "C" int fo_gemm_signal_noalloc(const fo_plan *p, const void *A, const void *B, void *reorder_buf,
                                      uint32_t **sig_out, uint32_t *epoch_out, hipStream_t stream) {
  if (!p || p->host_only || !p->dev_block || !sig_out || !epoch_out) return FO_ERR_INVALID;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != p->device) return FO_ERR_INVALID;
  if (dev < 0 || dev >= kMaxDevices) return FO_ERR_UNSUPPORTED;
  if (p->sig_words() > kStaticSigWords) return FO_ERR_UNSUPPORTED;
  if (p->NT > 0) {
    if (!A || !B || (reinterpret_cast<uintptr_t>(A) & 15u) || (reinterpret_cast<uintptr_t>(B) & 15u))
      return FO_ERR_INVALID;
    if (p->M * p->N > 0 && (!reorder_buf || (reinterpret_cast<uintptr_t>(reorder_buf) & 15u)))
      return FO_ERR_INVALID;
  }
  uint32_t *sig = nullptr;
  uint32_t epoch = 0;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
      void *ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FO_ERR_HIP;
      g_scratch[dev] = static_cast<uint32_t *>(ptr);
    }
    sig = g_scratch[dev];
    epoch = ++g_epoch[dev];
    if (epoch == 0) epoch = ++g_epoch[dev];  // epochs are never 0
  }
  *sig_out = sig;
  *epoch_out = epoch;
  if (p->NT == 0) return FO_OK;
  const int32_t words = p->sig_words();
  hipLaunchKernelGGL(clear_words, dim3((words + 255) / 256), dim3(256), 0, stream, sig, words);
  if (hipGetLastError() != hipSuccess) return FO_ERR_HIP;
  return fo::launch_gemm(p, A, B, reorder_buf, false, sig, epoch, nullptr, nullptr, stream, true);
}
