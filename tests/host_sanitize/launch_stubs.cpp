// Stand-ins for the kernel launchers, for the host-only sanitizer build of
// libfo (tests/test_host_sanitizers.py): the planner, the search and the
// argument checks of the C ABI are compiled with AddressSanitizer and
// UndefinedBehaviorSanitizer by the host compiler, and every launch reports
// FO_ERR_UNSUPPORTED.  No GPU code is built or run.
#include "../../gemm_tile_signaling_amd/csrc/fo_internal.h"

namespace fo {

int launch_gemm(const fo_plan *, const void *, const void *, void *, bool, uint32_t *, uint32_t, uint64_t *,
                uint32_t *, hipStream_t, bool) {
  return FO_ERR_UNSUPPORTED;
}
int launch_consume(const fo_plan *, const void *, const void *, void *, const uint32_t *, uint32_t, int32_t, int32_t,
                   int32_t *, uint64_t, int32_t, uint64_t *, hipStream_t) {
  return FO_ERR_UNSUPPORTED;
}
int launch_consume_ready(const fo_plan *, const void *, const void *, void *, const uint32_t *, uint32_t, int32_t,
                         int32_t *, uint64_t *, hipStream_t) {
  return FO_ERR_UNSUPPORTED;
}
int launch_shards(const fo_plan *, const void *, void *, hipStream_t) { return FO_ERR_UNSUPPORTED; }
int launch_row_exchange(const fo_plan *, const void *, void *, const void *, int, hipStream_t) {
  return FO_ERR_UNSUPPORTED;
}
int launch_reorder(const fo_plan *, const void *, void *, bool, int32_t, int32_t, hipStream_t) {
  return FO_ERR_UNSUPPORTED;
}
int launch_post_ep(const fo_plan *, const void *, void *, const void *, int, hipStream_t) { return FO_ERR_UNSUPPORTED; }
int launch_mfma_rate(int, const void *, int64_t, int32_t, int32_t, float *, hipStream_t) { return FO_ERR_UNSUPPORTED; }

}  // namespace fo

extern "C" int fo_gemm_signal_noalloc(const fo_plan *, const void *, const void *, void *, uint32_t **, uint32_t *,
                                      hipStream_t) {
  return FO_ERR_UNSUPPORTED;
}
