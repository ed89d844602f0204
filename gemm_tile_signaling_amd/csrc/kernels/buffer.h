// Buffer-resource construction shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fo {

// Word 3 of a raw (unswizzled, stride 0) buffer resource with a 32-bit data
// format; with stride 0 the range check compares byte offsets against
// `num_records`, so an access at or past `bytes` loads zeros and drops stores.
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Buffer resource for `bytes` bytes at `base`.  Both are the same in every lane;
// saying so keeps the resource in scalar registers (a resource the compiler
// thinks may vary per lane turns every buffer access into a loop over lanes).
// readfirstlane returns a signed int: both halves go through uint32_t before
// they are widened, or a low word with bit 31 set would sign-extend into the
// high word and point the resource outside the allocation.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void *ub = reinterpret_cast<void *>(((uint64_t)hi << 32) | (uint64_t)lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

}  // namespace fo
