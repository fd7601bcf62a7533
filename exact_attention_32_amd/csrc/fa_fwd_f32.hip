// fa_fwd_f32.hip -- fused attention forward for gfx950 with fp32 inputs,
// output and arithmetic (no value is rounded to a narrower type).
//
// Same operation and the same online-softmax recurrence as the bf16 kernel
// (page "解析 FlashAttention（2）", eq. (17), (20), (36)-(37), unnormalised
// form with one division at the end; query tiles outside, key/value tiles
// inside), but on the vector ALUs: each thread owns one query row, its q
// vector and its fp32 output accumulator live in registers, and 32-key tiles
// of K and V are staged in LDS and read by all threads as broadcasts.
// This path serves fp32 callers and small problems; it is not tuned.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kRows = 128;  // query rows (= threads) per workgroup

// Keys per LDS tile: 32 at d = 64; 16 at d = 128 so that q, the accumulator
// and the tile's scores fit the 256 vector registers without spilling.
template <int D>
constexpr int tile_keys() { return D >= 96 ? 16 : 32; }

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kRows)
fwd_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
               const float *__restrict__ V, float *__restrict__ O, float *__restrict__ LSE,
               int N, int nqt, float scale, float scale_log2) {
    constexpr int kTile = tile_keys<D>();
    __shared__ __attribute__((aligned(16))) float ks[kTile * D];
    __shared__ __attribute__((aligned(16))) float vs[kTile * D];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x / nqt;
    const int qt = blockIdx.x - bh * nqt;
    const int r0 = qt * kRows;
    const int qrow = r0 + tid;
    const size_t hoff = (size_t)bh * (size_t)N * D;

    float q[D];
#pragma unroll
    for (int t = 0; t < D; t += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (qrow < N) x = *reinterpret_cast<const float4 *>(Q + hoff + (size_t)qrow * D + t);
        q[t] = x.x; q[t + 1] = x.y; q[t + 2] = x.z; q[t + 3] = x.w;
    }
    float acc[D];
#pragma unroll
    for (int t = 0; t < D; ++t) acc[t] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int kv_end = CAUSAL ? min(N, r0 + kRows) : N;
    for (int c0 = 0; c0 < kv_end; c0 += kTile) {
        __syncthreads();  // previous tile fully consumed
        for (int u = tid; u < kTile * D / 4; u += kRows) {
            const int row = u / (D / 4);
            const int c = u - row * (D / 4);
            const int key = c0 + row;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < N) {
                kx = *reinterpret_cast<const float4 *>(K + hoff + (size_t)key * D + 4 * c);
                vx = *reinterpret_cast<const float4 *>(V + hoff + (size_t)key * D + 4 * c);
            }
            *reinterpret_cast<float4 *>(&ks[row * D + 4 * c]) = kx;
            *reinterpret_cast<float4 *>(&vs[row * D + 4 * c]) = vx;
        }
        __syncthreads();

        // Scores of this tile, masked keys set to -inf.
        float s[kTile];
        float mt = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < kTile; ++kk) {
            float dot = 0.f;
#pragma unroll
            for (int t = 0; t < D; t += 4) {
                const float4 kx = *reinterpret_cast<const float4 *>(&ks[kk * D + t]);
                dot = fmaf(q[t], kx.x, dot);
                dot = fmaf(q[t + 1], kx.y, dot);
                dot = fmaf(q[t + 2], kx.z, dot);
                dot = fmaf(q[t + 3], kx.w, dot);
            }
            const int key = c0 + kk;
            const bool hidden = key >= N || (CAUSAL && key > qrow);
            s[kk] = hidden ? -INFINITY : dot;
            mt = fmaxf(mt, s[kk]);
        }
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f((m_run - m_use) * scale_log2);  // from the old max
        const float mc = m_use * scale_log2;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < D; ++t) acc[t] *= alpha;  // rescale before adding
#pragma unroll
        for (int kk = 0; kk < kTile; ++kk) {
            const float p = exp2f(fmaf(s[kk], scale_log2, -mc));
            l_run += p;
#pragma unroll
            for (int t = 0; t < D; t += 4) {
                const float4 vx = *reinterpret_cast<const float4 *>(&vs[kk * D + t]);
                acc[t] = fmaf(p, vx.x, acc[t]);
                acc[t + 1] = fmaf(p, vx.y, acc[t + 1]);
                acc[t + 2] = fmaf(p, vx.z, acc[t + 2]);
                acc[t + 3] = fmaf(p, vx.w, acc[t + 3]);
            }
        }
        m_run = m_new;
    }

    if (qrow < N) {
        const float inv = 1.f / l_run;
        float *orow = O + hoff + (size_t)qrow * D;
#pragma unroll
        for (int t = 0; t < D; t += 4)
            *reinterpret_cast<float4 *>(orow + t) =
                make_float4(acc[t] * inv, acc[t + 1] * inv, acc[t + 2] * inv, acc[t + 3] * inv);
        LSE[(size_t)bh * N + qrow] = m_run * scale + logf(l_run);
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const float *q, const float *k, const float *v, float *o, float *lse, int B,
                  int H, int N, float scale, hipStream_t stream) {
    const int nqt = (N + kRows - 1) / kRows;
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(B * H * nqt), dim3(kRows), 0, stream, q,
                       k, v, o, lse, N, nqt, scale, scale_log2);
    return hipGetLastError();
}

}  // namespace

template <int D>
hipError_t launch_c(const float *q, const float *k, const float *v, float *o, float *lse, int B,
                    int H, int N, float scale, bool causal, hipStream_t stream) {
    return causal ? launch<D, true>(q, k, v, o, lse, B, H, N, scale, stream)
                  : launch<D, false>(q, k, v, o, lse, B, H, N, scale, stream);
}

hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                          int B, int H, int N, int d, float scale, bool causal,
                          hipStream_t stream) {
    switch (d) {
        case 16: return launch_c<16>(q, k, v, o, lse, B, H, N, scale, causal, stream);
        case 32: return launch_c<32>(q, k, v, o, lse, B, H, N, scale, causal, stream);
        case 48: return launch_c<48>(q, k, v, o, lse, B, H, N, scale, causal, stream);
        case 64: return launch_c<64>(q, k, v, o, lse, B, H, N, scale, causal, stream);
        case 80: return launch_c<80>(q, k, v, o, lse, B, H, N, scale, causal, stream);
        case 96: return launch_c<96>(q, k, v, o, lse, B, H, N, scale, causal, stream);
        case 112: return launch_c<112>(q, k, v, o, lse, B, H, N, scale, causal, stream);
        default: return launch_c<128>(q, k, v, o, lse, B, H, N, scale, causal, stream);
    }
}

}  // namespace fa
