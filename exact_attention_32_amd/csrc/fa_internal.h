// fa_internal.h -- declarations shared by the C-ABI front end (fa_api.cpp) and
// the kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

// FA_SAFE_SYNC=1 builds a checking variant of the library: every copy into
// an LDS tile buffer is completed and made visible by a workgroup barrier
// before any wave computes on, and every buffer's reads complete at a barrier
// before it is refilled.  Its results must equal the regular build's bit for
// bit (the arithmetic is unchanged; only the overlap of copies and compute
// goes); a difference would show a missing wait or barrier in the regular
// pipelines.
#ifndef FA_SAFE_SYNC
#define FA_SAFE_SYNC 0
#endif

namespace fa {

constexpr bool kSafeSync = FA_SAFE_SYNC != 0;

// Compute units of the current device (looked up once per device; 256 if
// the runtime cannot say).
int device_cus();

// Each launcher enqueues one kernel on `stream` and returns the launch status
// (hipGetLastError).  Arguments have already been validated by fa_api.cpp.
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o,
                           float *lse, int B, int H, int N, int d, float scale,
                           bool causal, hipStream_t stream);

// bf16 (fp16 = false) or fp16 views with element strides (q, k, v, o: batch,
// head, row; d contiguous); the dense layout takes the contiguous kernels.
hipError_t launch_fwd_ex(bool fp16, const void *q, const void *k, const void *v, void *o,
                         float *lse, int B, int H, int N, int d, float scale, bool causal,
                         const int64_t *strides, hipStream_t stream);

hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o,
                          float *lse, int B, int H, int N, int d, float scale,
                          bool causal, hipStream_t stream);

// Backward pass: enqueues the dq kernel (which also writes delta) and then the
// dkdv kernel on `stream`.
hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const void *dout, const float *lse, void *dq, void *dk, void *dv,
                           float *delta, int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream);

// The backward pass on bf16 (fp16 = false) or fp16 views with element
// strides (q, k, v, o, dout, dq, dk, dv: batch, head, row; d contiguous);
// lse and delta dense.  The dense layout takes the contiguous kernels.
hipError_t launch_bwd_ex(bool fp16, const void *q, const void *k, const void *v, const void *o,
                         const void *dout, const float *lse, void *dq, void *dk, void *dv,
                         float *delta, int B, int H, int N, int d, float scale, bool causal,
                         const int64_t *strides, hipStream_t stream);

// Forward pass in the key/value-outer order of Algorithm 1: one launch per
// 64-key block; ows [B,H,N,d], lws, mws [B,H,N] (fp32) carry O, l, m between
// launches.
hipError_t launch_fwd_kvouter_bf16(const void *q, const void *k, const void *v, void *o,
                                   float *lse, int B, int H, int N, int d, float scale,
                                   bool causal, float *ows, float *lws, float *mws,
                                   hipStream_t stream);

// Decode (few queries over many keys, key axis split in chunks).
constexpr int kDecodeMaxQueries = 16;
// Bytes of the fixed device scratch of fa_decode_noalloc (the partial outputs
// and LSEs of the automatic split count at B2 H32 Nq16 d128 fit).
constexpr unsigned long kDecodeScratchBytes = FA_DECODE_SCRATCH_BYTES;
static_assert(kDecodeScratchBytes % 256 == 0, "scratch size");
constexpr int kMaxDevices = 64;
// Device address of the current device's copy of that scratch (looked up
// once per device with hipGetSymbolAddress).
hipError_t decode_scratch(void **ptr);
constexpr int kDecodeMinChunk = 64;  // keys per chunk, at least
// At most this many queries run on the vector-ALU kernels, more on the MFMA
// kernel.
constexpr int kDecodeValuQueries = 2;
// Single-wave workgroups aimed for by the automatic split count (sized for
// 256 compute units): the vector-ALU kernels, 8 per compute unit; the MFMA
// kernel, whose three 16 KiB tile buffers per wave leave room for three
// waves per compute unit at d = 128, one round of them (a second, partial
// round of waves costs more than the longer chunks: B2 H32 Nq16 Nk8192 d128
// causal 47 us at 704 waves against 54-56 us at 960-2048).
constexpr int kDecodeTargetWaves = 2048;
constexpr int kDecodeTargetWavesMfma = 768;
// Number of chunks for a requested count (<= 0: automatic).
int decode_num_splits(int B, int H, int Nq, int Nk, int requested);
// Keys per chunk for S chunks: the least multiple of `granule` that covers
// Nk in S chunks (the kernels' unit of work: 64 keys for the vector-ALU
// kernels, whole blocks of loads at both head dims; 96 for the MFMA kernel,
// one round of three 32-key tiles).
int decode_chunk(int Nk, int S, int granule);
// Enqueues the split kernel (partials into o_part [B,H,S,Nq,d] and lse_part
// [B,H,S,Nq], fp32) and the merge kernel.
hipError_t launch_decode_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                              int B, int H, int Nq, int Nk, int d, float scale, bool causal,
                              int S, float *o_part, float *lse_part, hipStream_t stream);
// The same on bf16 (fp16 = false) or fp16 views with element strides (q, k,
// v, o: batch, head, row; d contiguous); the dense layout takes the
// contiguous kernels.
hipError_t launch_decode_ex(bool fp16, const void *q, const void *k, const void *v, void *o,
                            float *lse, int B, int H, int Nq, int Nk, int d, float scale,
                            bool causal, int S, float *o_part, float *lse_part,
                            const int64_t *strides, hipStream_t stream);

}  // namespace fa
