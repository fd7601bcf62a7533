// fa_fwd_bf16.hip -- fused attention forward for gfx950, bf16 in / bf16 out,
// fp32 scores, softmax statistics and accumulator.
//
// What is computed: O = softmax(scale * Q K^T [+ causal mask]) V per
// (batch, head), with the per-row log-sum-exp, as defined on the page
// "解析 FlashAttention（2）" (section 1.1; safe softmax eq. (2)-(5)).  The
// tile-by-tile schedule is the online-softmax recurrence of the same page
// (eq. (17), (20) for the statistics, eq. (36)-(37) for the output), written
// in the unnormalised form with one division at the end and with query tiles
// outside / key-value tiles inside, as in the FlashAttention-2 loop of the
// unit-12 lesson "在线 Softmax 与 FlashAttention" (loop-order part), which
// states both orders give the same result.
//
// Mapping onto CDNA4
// ------------------
// * One workgroup = 4 wavefronts = 128 query rows of one (batch, head); each
//   wave owns 32 rows for the whole key loop (Q, the output accumulator and
//   the running max / sum never leave registers).
// * Key/value tiles of 64 keys are staged global -> registers -> LDS with
//   16-byte loads, double-buffered: the loads of tile t+1 are issued before
//   the matrix work of tile t and written to the other LDS buffer after it.
// * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: with K as the A operand and Q^T
//   as the B operand, lane (g, j) of the accumulator holds query j and 16 of
//   the 32 keys of a block, so a row's max and sum are in-register reductions
//   plus one exchange between the two half-waves.
// * O^T += V^T P^T on the same instruction: the probabilities leave the S
//   accumulator already in the B-operand layout of this product (the 16
//   accumulator rows of a lane are taken as the K index of the next MFMA),
//   so P never goes through LDS.  V is transposed while it is staged into
//   LDS, with the key order inside each 16-key group permuted to match.
// * Causal: key tiles wholly in the future of the workgroup are never loaded
//   (loop bound), a wave whose 32 rows are all before a tile skips its math,
//   and only tiles that straddle the diagonal (or the ragged end of N) pay
//   for the element-wise mask (unit-12 causal-mask lesson: skip / diagonal /
//   past tiles).
// * The running maximum is kept per row; the accumulator is rescaled by
//   alpha = e^(m_old - m_new) only when some row's maximum moved (the factor
//   is exactly 1 otherwise).
// * Grid: workgroups are dealt round-robin over the 8 XCDs; consecutive
//   workgroup ids are remapped so that each XCD walks a contiguous range of
//   heads (its 4 MB L2 then serves the K/V stream of one head to all its
//   query tiles).  Under the causal mask the longest query tiles of a head
//   are issued first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 32;
constexpr int kBr = 4 * kRowsPerWave;  // query rows per workgroup
constexpr int kBc = 64;                // keys per tile

// Shared-memory tiles, unpadded; 16-byte chunks are XOR-swizzled by row so
// that both the staging writes and the MFMA operand reads spread over the
// LDS banks.
//   K tile : [kBc keys][D], chunk c of row r lives at chunk c ^ (r & 7).
//   Vt tile: [D][kBc keys, permuted], chunk c of row r at c ^ ((r ^ r>>3) & 7).
template <int D>
struct Tiles {
    __bf16 k[2][kBc * D];
    __bf16 vt[2][D * kBc];
};

template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {
    return row * D + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ int vt_off(int row, int chunk) {
    return row * kBc + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 3);
}

// Position of key x (0..kBc-1) inside a transposed V row: bits 2 and 3 of the
// key index are swapped, so that the 8 keys one lane feeds to the PV MFMA
// (keys 16t + 4g + {0..3} and 16t + 8 + 4g + {0..3}) are contiguous.
__device__ __forceinline__ int key_perm(int x) {
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Workgroup id -> (batch*head, query tile).  Consecutive ids go to
// consecutive XCDs; when the grid divides evenly, XCD x receives the
// contiguous range [x*W/8, (x+1)*W/8) of (head, tile) pairs.
__device__ __forceinline__ void map_block(int L, int W, int nqt, bool heavy_first,
                                          int &bh, int &qt) {
    int gidx = L;
    if ((W & 7) == 0) {
        const int per = W >> 3;
        gidx = (L & 7) * per + (L >> 3);
    }
    bh = gidx / nqt;
    qt = gidx - bh * nqt;
    if (heavy_first) qt = nqt - 1 - qt;
}

__device__ __forceinline__ u32x4 load16(const __bf16 *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K,
                const __bf16 *__restrict__ V, __bf16 *__restrict__ O,
                float *__restrict__ LSE, int N, int nqt, float scale, float scale_log2) {
    static_assert(D == 64 || D == 128, "head dim");
    __shared__ __attribute__((aligned(16))) Tiles<D> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 5;  // half-wave
    const int j = lane & 31;  // query column of this lane

    int bh, qt;
    map_block(blockIdx.x, gridDim.x, nqt, CAUSAL, bh, qt);
    const int r0 = qt * kBr;
    const size_t hoff = (size_t)bh * (size_t)N * D;
    const __bf16 *Qh = Q + hoff;
    const __bf16 *Kh = K + hoff;
    const __bf16 *Vh = V + hoff;
    const int wrow0 = r0 + wave * kRowsPerWave;
    const int qrow = wrow0 + j;

    // Q^T as the B operand: lane (g, j) holds query qrow, columns 16ks+8g..+7.
    bf16x8 qop[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qrow < N) x = load16(Qh + (size_t)qrow * D + 16 * ks + 8 * g);
        qop[ks] = __builtin_bit_cast(bf16x8, x);
    }

    const int kv_end = CAUSAL ? min(N, r0 + kBr) : N;
    const int n_tiles = (kv_end + kBc - 1) / kBc;

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m_run = -INFINITY;  // running max of the raw scores of row qrow
    float l_run = 0.f;        // this half-wave's share of the running sum

    // ---- staging: global -> registers -> LDS ------------------------------
    constexpr int kKChunks = kBc * D / 8 / kThreads;  // 16-byte K chunks per thread
    constexpr int kVUnits = (kBc / 4) * (D / 8);      // 4-key x 8-column V blocks
    u32x4 kreg[kKChunks];
    u32x4 vreg[4];

    auto load_tile = [&](int c0) {
#pragma unroll
        for (int u = 0; u < kKChunks; ++u) {
            const int chunk = tid + kThreads * u;
            const int row = chunk / (D / 8);
            const int c = chunk % (D / 8);
            const int key = c0 + row;
            kreg[u] = u32x4{0u, 0u, 0u, 0u};
            if (key < N) kreg[u] = load16(Kh + (size_t)key * D + c * 8);
        }
        if (tid < kVUnits) {
            const int c = tid % (D / 8);
            const int kq = tid / (D / 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = c0 + 4 * kq + e;
                vreg[e] = u32x4{0u, 0u, 0u, 0u};
                if (key < N) vreg[e] = load16(Vh + (size_t)key * D + c * 8);
            }
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kKChunks; ++u) {
            const int chunk = tid + kThreads * u;
            const int row = chunk / (D / 8);
            const int c = chunk % (D / 8);
            *reinterpret_cast<u32x4 *>(&sm.k[buf][k_off<D>(row, c)]) = kreg[u];
        }
        if (tid < kVUnits) {
            // vreg[e] = V[4kq+e][8c .. 8c+7]; dword h holds columns 8c+2h (low
            // half) and 8c+2h+1 (high half).  Write column 8c+2h (+1) of the
            // four keys as one 8-byte row segment of the transposed tile.
            const int c = tid % (D / 8);
            const int kq = tid / (D / 8);
            const int col = key_perm(4 * kq);
            const int chunk = col >> 3;
            const int half = (col >> 2) & 1;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t a0 = vreg[0][h], a1 = vreg[1][h];
                const uint32_t a2 = vreg[2][h], a3 = vreg[3][h];
                u32x2 lo, hi;
                lo[0] = (a0 & 0xffffu) | (a1 << 16);
                lo[1] = (a2 & 0xffffu) | (a3 << 16);
                hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                const int row = 8 * c + 2 * h;
                *reinterpret_cast<u32x2 *>(&sm.vt[buf][vt_off(row, chunk) + 4 * half]) = lo;
                *reinterpret_cast<u32x2 *>(&sm.vt[buf][vt_off(row + 1, chunk) + 4 * half]) = hi;
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        const int c0 = t * kBc;
        const bool has_next = t + 1 < n_tiles;
        if (has_next) load_tile(c0 + kBc);

        // A wave whose rows all precede this tile has nothing to add.
        const bool active = !CAUSAL || c0 <= wrow0 + kRowsPerWave - 1;
        if (active) {
            const __bf16 *kt = sm.k[buf];
            const __bf16 *vt = sm.vt[buf];

            // S^T[key][query] = K Q^T for the kBc keys of this tile.
            f32x16 s[kBc / 32];
#pragma unroll
            for (int kb = 0; kb < kBc / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        kt + k_off<D>(32 * kb + j, 2 * ks + g));
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[ks], s[kb], 0, 0, 0);
                }
            }

            // Element r of s[kb] is key c0 + 32kb + 8(r/4) + 4g + r%4.
            const bool need_mask = (CAUSAL && c0 + kBc - 1 > wrow0) || (c0 + kBc > N);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < kBc / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = c0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                        const bool hidden = key >= N || (CAUSAL && key > qrow);
                        if (hidden) s[kb][r] = -INFINITY;
                    }
            }

            // Tile row maximum: in-register, then across the two half-waves.
            float mt = s[0][0];
#pragma unroll
            for (int kb = 0; kb < kBc / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            // A row that has seen no visible key keeps base 0 (its terms are 0).
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            // alpha from the OLD maximum, before it is replaced.
            const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
            const float mc = m_use * scale_log2;

            // P = exp(scale*(s - m)) = 2^(s*scale*log2e - m*scale*log2e).
            bf16x8 pop[kBc / 16];
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < kBc / 32; ++kb) {
                f32x8 lo, hi;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    lo[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], scale_log2, -mc));
                    hi[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 8], scale_log2, -mc));
                    rs += lo[r];
                    rs += hi[r];
                }
                pop[2 * kb] = __builtin_convertvector(lo, bf16x8);
                pop[2 * kb + 1] = __builtin_convertvector(hi, bf16x8);
            }
            l_run = l_run * alpha + rs;
            // Rescale the accumulator first, then add this tile's P V.
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            }
            m_run = m_new;

            // O^T[d][query] += V^T P^T; k-step T covers keys 16T..16T+15.
#pragma unroll
            for (int T = 0; T < kBc / 16; ++T)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        vt + vt_off(32 * db + j, 2 * T + g));
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[T], acc[db], 0, 0, 0);
                }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: O = acc / l, rounded to bf16; LSE = m*scale + ln(l).
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (qrow < N) {
        __bf16 *orow = O + hoff + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * a + e] * inv;
                *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * a + 4 * g) =
                    __builtin_convertvector(x, bf16x4);
            }
        if (g == 0) LSE[(size_t)bh * N + qrow] = m_run * scale + logf(l_tot);
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, void *o, float *lse,
                  int B, int H, int N, float scale, hipStream_t stream) {
    const int nqt = (N + kBr - 1) / kBr;
    const int blocks = B * H * nqt;
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k),
                       static_cast<const __bf16 *>(v), static_cast<__bf16 *>(o), lse, N, nqt,
                       scale, scale_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream) {
    if (d == 64)
        return causal ? launch<64, true>(q, k, v, o, lse, B, H, N, scale, stream)
                      : launch<64, false>(q, k, v, o, lse, B, H, N, scale, stream);
    return causal ? launch<128, true>(q, k, v, o, lse, B, H, N, scale, stream)
                  : launch<128, false>(q, k, v, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
