// fa_internal.h -- declarations shared by the C-ABI front end (fa_api.cpp) and
// the kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Each launcher enqueues one kernel on `stream` and returns the launch status
// (hipGetLastError).  Arguments have already been validated by fa_api.cpp.
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o,
                           float *lse, int B, int H, int N, int d, float scale,
                           bool causal, hipStream_t stream);

hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o,
                          float *lse, int B, int H, int N, int d, float scale,
                          bool causal, hipStream_t stream);

// Backward pass: enqueues the dq kernel (which also writes delta) and then the
// dkdv kernel on `stream`.
hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const void *dout, const float *lse, void *dq, void *dk, void *dv,
                           float *delta, int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream);

}  // namespace fa
