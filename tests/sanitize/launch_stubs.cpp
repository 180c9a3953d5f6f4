// Launch stubs for the host-only sanitizer build of the library (test infrastructure).
//
// The sanitizer build compiles the ABI layer (argument validation, launch planning,
// kernel-parameter packing), the mapper and the GOO planner for the host only, with
// AddressSanitizer and UndefinedBehaviorSanitizer, and links these stubs in place of
// the kernel launchers: every launch reports that no device is present, so a call
// that gets past validation fails loudly instead of computing anything.
#include <cstdint>

#include "ma_internal.h"

namespace ma {

namespace {
constexpr int kNoDevice = 100;  // hipErrorNoDevice
}

int launch_fwd_bf16(const FwdParams&, int, int, int, void*) { return kNoDevice; }
int launch_fwd_bf16_resident(const FwdParams&, int, int, void*) { return kNoDevice; }
int launch_fwd_f32(const FwdParams&, int, int, void*) { return kNoDevice; }
int launch_fill_empty(void*, float*, int, int, int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, void*) {
  return kNoDevice;
}
int launch_merge(const MergeParams&, int, int, void*) { return kNoDevice; }
int launch_reduce_add(const ReduceParams&, void*) { return kNoDevice; }
int launch_bwd_preprocess(const BwdPreParams&, int, void*) { return kNoDevice; }
int launch_bwd_dq(const BwdParams&, int, int, void*) { return kNoDevice; }
int launch_bwd_dkv(const BwdParams&, int, int, void*) { return kNoDevice; }

}  // namespace ma
