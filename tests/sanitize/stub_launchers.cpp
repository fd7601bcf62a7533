// Host-only stand-ins for the kernel launchers, for the sanitizer build of
// the C ABI's validation code (fa_api.cpp + fa_plan.cpp compiled by g++ with
// -fsanitize=address,undefined).  Every stub reports a failed launch; the
// checks that run under the sanitizers are the ones before any launch.
#include "fa_internal.h"

namespace fa {

hipError_t launch_fwd_bf16(const void *, const void *, const void *, void *, float *, int, int,
                           int, int, float, bool, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_fwd_ex(bool, const void *, const void *, const void *, void *, float *, int, int,
                         int, int, float, bool, const int64_t *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_fwd_f32(const float *, const float *, const float *, float *, float *, int, int,
                          int, int, float, bool, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_bwd_bf16(const void *, const void *, const void *, const void *, const void *,
                           const float *, void *, void *, void *, float *, int, int, int, int,
                           float, bool, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_bwd_ex(bool, const void *, const void *, const void *, const void *,
                         const void *, const float *, void *, void *, void *, float *, int, int,
                         int, int, float, bool, const int64_t *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_fwd_kvouter_bf16(const void *, const void *, const void *, void *, float *, int,
                                   int, int, int, float, bool, float *, float *, float *,
                                   hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_decode_bf16(const void *, const void *, const void *, void *, float *, int, int,
                              int, int, int, float, bool, int, float *, float *, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_decode_ex(bool, const void *, const void *, const void *, void *, float *, int,
                            int, int, int, int, float, bool, int, float *, float *,
                            const int64_t *, hipStream_t) {
    return hipErrorInvalidValue;
}

hipError_t decode_scratch(void **ptr) {
    *ptr = nullptr;
    return hipErrorInvalidValue;
}

}  // namespace fa
