// Host-only stand-ins for the kernel launchers of libpkv, for a build of the
// C ABI and the block manager under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  The tests that run
// against that build check argument validation, sizing and the block
// manager, none of which reaches a launch; a launch that does get here
// reports an error instead of computing anything.

#include "pkv_internal.h"

namespace pkv {

hipError_t launch_decode(const DecodeLaunch&, hipStream_t) { return hipErrorInvalidDeviceFunction; }

hipError_t launch_reshape_and_cache(const void*, const void*, int, void*, void*, int, float, float, const int64_t*,
                                    int, int, int, int, int, hipStream_t) {
  return hipErrorInvalidDeviceFunction;
}

hipError_t launch_copy_blocks(void*, void*, const void*, const void*, const int32_t*, int, int64_t, int, int,
                              hipStream_t) {
  return hipErrorInvalidDeviceFunction;
}

hipError_t static_workspace(hipStream_t, void**) { return hipErrorInvalidDeviceFunction; }

}  // namespace pkv
