// fa_fwd_f32.hip -- fused attention forward for gfx950 with fp32 inputs,
// output and arithmetic (no value is rounded to a narrower type).
//
// Same operation and the same online-softmax recurrence as the bf16 kernel
// (page "解析 FlashAttention（2）", eq. (17), (20), (36)-(37), unnormalised
// form with one division at the end), on the vector ALUs.  A workgroup takes
// R query rows and splits their key axis over S thread groups: thread
// (r, s) owns query row r and, in every 64-key tile staged in LDS, the keys
// s, s + S, ...; it keeps q, its own (m, l) and an unnormalised fp32
// accumulator in registers.  At the end the S partial results of a row are
// merged through LDS by the two-block rule of eq. (17)/(20) (each partial
// weighted by e^{m_s - m}), each thread producing D/S columns of the output.
// Splitting the keys puts S threads on every query row, so small problems
// spread over many more lanes than one thread per row would.  Two shapes of
// workgroup: R = 16 (8 above d = 64) rows and S = 16, and for grids that
// would leave compute units idle a quarter of the rows and S = 64 (four
// times the workgroups, a quarter of the keys per thread).  The S threads
// of a row are consecutive lanes, so a 16-lane pass of an LDS read fetches
// 16 different key rows (the pitch puts them in distinct banks) instead of
// broadcasting one.  This path serves fp32 callers and small problems; it
// is not a tuned hot path.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kTileKeys = 64;  // keys per LDS tile
// Query rows per workgroup of the default shape (S = 16): 16 (256 threads)
// up to d = 64, 8 (128 threads) above, where q and the accumulator take 2d
// registers per thread.
template <int D>
constexpr int kRowsF = D <= 64 ? 16 : 8;
// LDS row pitch in floats: 4 more than d, so that consecutive key rows start
// four banks apart.
template <int D>
constexpr int kPitch = D + 4;
// Floats of the shared array: the K and V tiles while the keys stream, then
// the partial results (acc, m, l) of every thread for the merge.
template <int D, int R, int S>
constexpr int kSharedFloats = 2 * kTileKeys * kPitch<D> > R * S * (D + 2)
                                  ? 2 * kTileKeys * kPitch<D>
                                  : R * S * (D + 2);

template <int D, int R, int kSplit, bool CAUSAL>
__global__ void __launch_bounds__(R * kSplit)
fwd_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
               const float *__restrict__ V, float *__restrict__ O, float *__restrict__ LSE,
               int N, int nqt, float scale, float scale_log2) {
    constexpr int kPerTile = kTileKeys / kSplit;  // keys per thread and tile
    constexpr int P = kPitch<D>;
    constexpr int kThreadsF = R * kSplit;
    __shared__ __attribute__((aligned(16))) float sh[kSharedFloats<D, R, kSplit>];
    float *const ks = sh;                    // [kTileKeys][P]
    float *const vs = sh + kTileKeys * P;    // [kTileKeys][P]

    const int tid = threadIdx.x;
    const int r = tid / kSplit;
    const int sg = tid % kSplit;
    const int bh = blockIdx.x / nqt;
    const int qt = blockIdx.x - bh * nqt;
    const int r0 = qt * R;
    const int qrow = r0 + r;
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

    const int kv_end = CAUSAL ? min(N, r0 + R) : N;
    // Each thread copies kCopies float4 of K and of V per tile.  Up to
    // d = 64 (four each) the next tile's are loaded into registers before
    // this tile's compute, so that their latency overlaps it; above, the
    // registers are taken by q and the accumulator, and a tile is loaded
    // right before its use.
    constexpr int kCopies = kTileKeys * D / 4 / kThreadsF;
    static_assert(kCopies * kThreadsF == kTileKeys * D / 4, "tile copy split");
    constexpr bool kPrefetch = kCopies <= 4;
    float4 kn[kPrefetch ? kCopies : 1], vn[kPrefetch ? kCopies : 1];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int i = 0; i < (kPrefetch ? kCopies : 0); ++i) {
            const int u = tid + i * kThreadsF;
            const int row = u / (D / 4);
            const int c = u - row * (D / 4);
            const int key = c0 + row;
            kn[i] = vn[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (key < N) {
                kn[i] = *reinterpret_cast<const float4 *>(K + hoff + (size_t)key * D + 4 * c);
                vn[i] = *reinterpret_cast<const float4 *>(V + hoff + (size_t)key * D + 4 * c);
            }
        }
    };
    if constexpr (kPrefetch) {
        if (kv_end > 0) fetch(0);
    }
    for (int c0 = 0; c0 < kv_end; c0 += kTileKeys) {
        __syncthreads();  // previous tile fully consumed
#pragma unroll
        for (int i = 0; i < kCopies; ++i) {
            const int u = tid + i * kThreadsF;
            const int row = u / (D / 4);
            const int c = u - row * (D / 4);
            float4 kx, vx;
            if constexpr (kPrefetch) {
                kx = kn[i];
                vx = vn[i];
            } else {
                const int key = c0 + row;
                kx = vx = make_float4(0.f, 0.f, 0.f, 0.f);
                if (key < N) {
                    kx = *reinterpret_cast<const float4 *>(K + hoff + (size_t)key * D + 4 * c);
                    vx = *reinterpret_cast<const float4 *>(V + hoff + (size_t)key * D + 4 * c);
                }
            }
            *reinterpret_cast<float4 *>(&ks[row * P + 4 * c]) = kx;
            *reinterpret_cast<float4 *>(&vs[row * P + 4 * c]) = vx;
        }
        __syncthreads();
        if constexpr (kPrefetch) {
            if (c0 + kTileKeys < kv_end) fetch(c0 + kTileKeys);
        }

        // Scores of this thread's keys c0 + sg + kSplit j, masked keys -inf.
        float s[kPerTile];
        float mt = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < kPerTile; ++jj) {
            const int row = kSplit * jj + sg;
            float dot = 0.f;
#pragma unroll
            for (int t = 0; t < D; t += 4) {
                const float4 kx = *reinterpret_cast<const float4 *>(&ks[row * P + t]);
                dot = fmaf(q[t], kx.x, dot);
                dot = fmaf(q[t + 1], kx.y, dot);
                dot = fmaf(q[t + 2], kx.z, dot);
                dot = fmaf(q[t + 3], kx.w, dot);
            }
            const int key = c0 + row;
            const bool hidden = key >= N || (CAUSAL && key > qrow);
            s[jj] = hidden ? -INFINITY : dot;
            mt = fmaxf(mt, s[jj]);
        }
        // No visible key yet (m = -inf): exponents against 0, so that masked
        // scores give p = 0 and a NaN score still reaches l and acc.
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f((m_run - m_use) * scale_log2);  // from the old max
        const float mc = m_use * scale_log2;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < D; ++t) acc[t] *= alpha;  // rescale before adding
#pragma unroll
        for (int jj = 0; jj < kPerTile; ++jj) {
            const int row = kSplit * jj + sg;
            const float p = exp2f(fmaf(s[jj], scale_log2, -mc));
            l_run += p;
#pragma unroll
            for (int t = 0; t < D; t += 4) {
                const float4 vx = *reinterpret_cast<const float4 *>(&vs[row * P + t]);
                acc[t] = fmaf(p, vx.x, acc[t]);
                acc[t + 1] = fmaf(p, vx.y, acc[t + 1]);
                acc[t + 2] = fmaf(p, vx.z, acc[t + 2]);
                acc[t + 3] = fmaf(p, vx.w, acc[t + 3]);
            }
        }
        m_run = m_new;
    }

    // Merge the kSplit partials of each row: partial (r, sg) at
    // part[(r * kSplit + sg) * (D + 2)]: acc[0 .. D-1], m, l.
    __syncthreads();  // the tiles are no longer read
    float *const part = sh;
    {
        float *mine = part + (size_t)(r * kSplit + sg) * (D + 2);
#pragma unroll
        for (int t = 0; t < D; ++t) mine[t] = acc[t];
        mine[D] = m_run;
        mine[D + 1] = l_run;
    }
    __syncthreads();
    const float *rowp = part + (size_t)r * kSplit * (D + 2);
    float m_tot = -INFINITY;
#pragma unroll
    for (int g = 0; g < kSplit; ++g) m_tot = fmaxf(m_tot, rowp[g * (D + 2) + D]);
    float w[kSplit];
    float l_tot = 0.f;
#pragma unroll
    for (int g = 0; g < kSplit; ++g) {
        // a group that saw no visible key has m = -inf, l = 0: weight 0
        w[g] = exp2f((rowp[g * (D + 2) + D] - m_tot) * scale_log2);
        l_tot = fmaf(w[g], rowp[g * (D + 2) + D + 1], l_tot);
    }
    if (qrow < N) {
        const float inv = 1.f / l_tot;
        float *orow = O + hoff + (size_t)qrow * D;
        // columns sg, sg + 16, ... of the row
#pragma unroll
        for (int t = sg; t < D; t += kSplit) {
            float o = 0.f;
#pragma unroll
            for (int g = 0; g < kSplit; ++g) o = fmaf(w[g], rowp[g * (D + 2) + t], o);
            orow[t] = o * inv;
        }
        if (sg == 0) LSE[(size_t)bh * N + qrow] = m_tot * scale + logf(l_tot);
    }
}

template <int D, int R, int S, bool CAUSAL>
hipError_t launch_rs(const float *q, const float *k, const float *v, float *o, float *lse, int B,
                     int H, int N, float scale, hipStream_t stream) {
    const int nqt = (N + R - 1) / R;
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipLaunchKernelGGL((fwd_f32_kernel<D, R, S, CAUSAL>), dim3(B * H * nqt), dim3(R * S), 0,
                       stream, q, k, v, o, lse, N, nqt, scale, scale_log2);
    return hipGetLastError();
}

// The default shape, unless its grid has fewer workgroups than the device
// has compute units: then four times as many workgroups of a quarter of the
// rows, each row's keys split 64 ways (w1's B1 H1 N256 d64: 9.1 instead of
// 14.8 us; from about two workgroups per compute unit on the default shape
// is faster).
template <int D, bool CAUSAL>
hipError_t launch(const float *q, const float *k, const float *v, float *o, float *lse, int B,
                  int H, int N, float scale, hipStream_t stream) {
    constexpr int R = kRowsF<D>;
    const long wgs = (long)B * H * ((N + R - 1) / R);
    if (wgs < device_cus())
        return launch_rs<D, R / 4, 64, CAUSAL>(q, k, v, o, lse, B, H, N, scale, stream);
    return launch_rs<D, R, 16, CAUSAL>(q, k, v, o, lse, B, H, N, scale, stream);
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
