// fa_bwd_bf16.hip -- backward pass of the fused attention for gfx950: Q, K,
// V, O, dO in and dQ, dK, dV out, all bf16 (fa_bwd) or all bf16 or fp16 as
// dense tensors or strided views (fa_bwd_ex); fp32 scores, probabilities and
// accumulators.
//
// What is computed: the gradients of O = softmax(scale * Q K^T [+ causal
// mask]) V for an output gradient dO.  The pages describe the backward pass
// only as recomputation: S and P are rebuilt tile by tile from Q, K and the
// row statistics the forward pass kept, never stored as N x N matrices
// ("解析 FlashAttention（2）", section 1.2 (3), and the note after Algorithm 1
// that m and l are kept for the backward pass; the unit-12 lesson on memory;
// the Triton page, section 5.1: dQ, dK and dV, blocked and accumulated online).
// The per-tile formulas are the chain rule through P = softmax(S):
//   P_ij  = exp(scale * q_i.k_j - LSE_i)         (LSE from the forward pass)
//   dP_ij = dO_i . v_j
//   D_i   = sum_j P_ij dP_ij = dO_i . O_i
//   dS_ij = P_ij (dP_ij - D_i)
//   dV_j += P_ij dO_i,  dK_j += scale dS_ij q_i,  dQ_i += scale dS_ij k_j
//
// Two kernels, both on v_mfma_f32_32x32x16_bf16 with the operand layouts of
// the forward kernel (a lane owns one query or one key of a 32 x 32 block):
//  * dq kernel (query tiles outside, key tiles inside, like the forward):
//    computes D_i for its rows first and stores it for the second kernel;
//    then per 64-key tile S^T = K Q^T and dP^T = V dO^T, dS^T, and
//    dQ^T += K^T dS^T, where K^T comes out of the K tile through the LDS
//    transpose read.
//  * dkdv kernel (key tiles outside, query tiles inside): per 64-query tile
//    S = Q K^T and dP = dO V^T (Q, dO from LDS, K, V in registers), then
//    dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read transposed.
// Staging is the forward's: 16-byte direct-to-LDS buffer loads, double
// buffered, rows past N arriving as zeros; every tile that is read both
// row-wise and transposed uses one XOR swizzle that keeps both read patterns
// free of bank conflicts.  Causal: key tiles wholly after a query tile (or
// query tiles wholly before a key tile) are never visited; only tiles that
// straddle the diagonal or the ragged end of N pay for the element mask.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// dq kernel: one workgroup = 128 queries of one (batch, head); wave w owns
// queries r0 + 32w .. +31 (lane (g, j) holds query j of the wave).
// ---------------------------------------------------------------------------
// Both kernels run two waves per SIMD (<= 256 registers per lane), but for
// the d = 64 dq kernel on shorter rows (three, see the launcher).  The
// dkdv kernel holds K, V and two accumulators in registers (192 of them at
// d = 128); there its two 32-query halves run as a loop, not unrolled, which
// keeps their live ranges apart (a few registers still go to scratch, which
// measured faster than one wave per SIMD).
//
// A head dim DH that is not 64 or 128 runs in the tile layout of the next of
// the two (D): S and dP take DH/16 k-steps, the tiles and the dQ, dK, dV
// accumulators have D/32 d-blocks, and only the first DH columns are
// stored; the tile columns at and past DH feed only the unstored rows.
template <int DH>
constexpr int kLayout = DH <= 64 ? 64 : 128;
template <int D>
constexpr int kDqWaves = 2;
template <int D>
constexpr int kDkdvWaves = 2;
// Rows shorter than this run the d = 64 dq kernel at three waves per SIMD.
constexpr int kDq3MaxN = 8192;

// Element strides (batch, head, row) of the eight [B, H, N, d] tensors, d
// contiguous, in the order of the enum below; LSE and delta stay dense
// [B, H, N].  Used by the STRIDED instantiations only (the dense ones form
// bh * N * d and d).
enum BwdTensor { kTQ, kTK, kTV, kTO, kTDO, kTDQ, kTDK, kTDV, kTensors };
struct BwdStrides {
    long long b[kTensors], h[kTensors];
    int n[kTensors];
    int H;
};

// Element offset of head bh of tensor t, and its row stride.
template <int DH, bool STRIDED>
__device__ __forceinline__ size_t head_offset(const BwdStrides &st, int bh, int N, int t) {
    if constexpr (STRIDED) {
        const int b = bh / st.H, h = bh - b * st.H;
        return (size_t)(b * st.b[t] + h * st.h[t]);
    } else {
        return (size_t)bh * (size_t)N * DH;
    }
}
template <int DH, bool STRIDED>
__device__ __forceinline__ int row_stride(const BwdStrides &st, int t) {
    if constexpr (STRIDED) return st.n[t];
    else return DH;
}

template <typename E, int DH, bool CAUSAL, bool STRIDED, int OCC = kDqWaves<kLayout<DH>>>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(OCC, OCC)))
bwd_dq_kernel(const E *__restrict__ Q, const E *__restrict__ K, const E *__restrict__ V,
              const E *__restrict__ O, const E *__restrict__ dO, const float *__restrict__ LSE,
              float *__restrict__ Delta, E *__restrict__ dQ, int N, int ntiles, float scale,
              float scale_log2, BwdStrides st) {
    typedef typename TileOps<E>::x8 X8;
    constexpr int D = kLayout<DH>;
    constexpr int KS = DH / 16;  // k-steps of S^T and dP^T
    __shared__ __attribute__((aligned(16))) __bf16 lds_k0[kInner * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_k1[kInner * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v0[kInner * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v1[kInner * D];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 5;
    const int j = lane & 31;

    int bh, qt;
    map_block(blockIdx.x, gridDim.x, ntiles, CAUSAL, CAUSAL, 64, bh, qt);  // 2 per CU
    const int r0 = qt * kOuter;
    const E *Kh = K + head_offset<DH, STRIDED>(st, bh, N, kTK);
    const E *Vh = V + head_offset<DH, STRIDED>(st, bh, N, kTV);
    const int kn = row_stride<DH, STRIDED>(st, kTK), vn = row_stride<DH, STRIDED>(st, kTV);
    const int wrow0 = r0 + wave * kRowsPerWave;
    const int qrow = wrow0 + j;
    const bool valid = qrow < N;

    // Q^T and dO^T as B operands: lane (g, j) holds columns 16ks+8g..+7 of
    // its query row.  D_i = dO_i . O_i from the same columns, then summed
    // over the two half-waves.
    const E *Qr = Q + head_offset<DH, STRIDED>(st, bh, N, kTQ) +
                  (size_t)qrow * row_stride<DH, STRIDED>(st, kTQ);
    const E *dOr = dO + head_offset<DH, STRIDED>(st, bh, N, kTDO) +
                   (size_t)qrow * row_stride<DH, STRIDED>(st, kTDO);
    const E *Or = O + head_offset<DH, STRIDED>(st, bh, N, kTO) +
                  (size_t)qrow * row_stride<DH, STRIDED>(st, kTO);
    X8 qop[KS], doop[KS];
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 xq = {0u, 0u, 0u, 0u}, xd = {0u, 0u, 0u, 0u}, xo = {0u, 0u, 0u, 0u};
        if (valid) {
            const int e = 16 * ks + 8 * g;
            xq = load16(Qr + e);
            xd = load16(dOr + e);
            xo = load16(Or + e);
        }
        qop[ks] = __builtin_bit_cast(X8, xq);
        doop[ks] = __builtin_bit_cast(X8, xd);
        const X8 ov = __builtin_bit_cast(X8, xo);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)doop[ks][e], (float)ov[e], dpart);
    }
    float delta;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dpart),
                                                         __float_as_uint(dpart), false, false);
        delta = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (valid && g == 0) Delta[(size_t)bh * N + qrow] = delta;
    const float lse2 = valid ? LSE[(size_t)bh * N + qrow] * kLog2e : 0.f;

    const int kv_end = CAUSAL ? min(N, r0 + kOuter) : N;
    const int n_tiles = (kv_end + kInner - 1) / kInner;

    // K and V may have different row strides in a strided call.
    const uint32_t ksrc = tile_src_offset<D, DH>(wave, lane, kn);
    const uint32_t vsrc = STRIDED ? tile_src_offset<D, DH>(wave, lane, vn) : ksrc;
    const uint32_t rd = row_read_offset<D>(lane);
    uint32_t trd[2];
    tr_read_offsets<D>(lane, trd);

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    LDS3 char *const k0 = (LDS3 char *)lds_k0;
    LDS3 char *const k1 = (LDS3 char *)lds_k1;
    LDS3 char *const v0 = (LDS3 char *)lds_v0;
    LDS3 char *const v1 = (LDS3 char *)lds_v1;

    auto step = [&](int t, const LDS3 char *kt, const LDS3 char *vt, LDS3 char *nk, LDS3 char *nv) {
        const int c0 = t * kInner;
        if (t + 1 < n_tiles) {
            load_tile<D, DH, STRIDED>(Kh, N, c0 + kInner, nk, ksrc, wave, kn);
            load_tile<D, DH, STRIDED>(Vh, N, c0 + kInner, nv, vsrc, wave, vn);
        }
        if constexpr (kSafeSync) {  // checking build: the copies land before any compute
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        const bool active = !CAUSAL || c0 <= wrow0 + kRowsPerWave - 1;
        if (active) {
            // Element r of s[kb] is key c0 + 32kb + 8(r/4) + 4g + r%4.
            const bool need_mask = (CAUSAL && c0 + kInner - 1 > wrow0) || (c0 + kInner > N);
            const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - c0 - 4 * g;
            f32x16 s[2], dp[2];
            X8 dsop[4];
            // S^T = K Q^T and dP^T = V dO^T for the 32 keys of block kb.
            auto products = [&](int kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint32_t a = row_read_at(rd, ks) + kb * 32 * D * 2;
                    const X8 kf = *reinterpret_cast<const LDS3 X8 *>(kt + a);
                    const X8 vf = *reinterpret_cast<const LDS3 X8 *>(vt + a);
                    s[kb] = TileOps<E>::mfma(kf, qop[ks], s[kb]);
                    dp[kb] = TileOps<E>::mfma(vf, doop[ks], dp[kb]);
                }
            };
            auto mask = [&](int kb) {
                if (need_mask) {
                    keep_branch();
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
                }
            };
            // dS^T = P^T o (dP^T - D) of block kb, rounded to bf16 as the B
            // operands of k-steps 2kb (rows 0-7) and 2kb + 1 (rows 8-15).
            auto dscores = [&](int kb) {
                f32x8 lo, hi;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const float plo = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], scale_log2, -lse2));
                    const float phi = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 8], scale_log2, -lse2));
                    lo[r] = plo * (dp[kb][r] - delta);
                    hi[r] = phi * (dp[kb][r + 8] - delta);
                }
                dsop[2 * kb] = __builtin_convertvector(lo, X8);
                dsop[2 * kb + 1] = __builtin_convertvector(hi, X8);
            };
            // dQ^T += K^T dS^T over k-steps T (keys 16T .. 16T + 15).
            auto dq_products = [&](int T) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = TileOps<E>::mfma(tr_read<D, X8>(kt, trd, T, db), dsop[T], acc[db]);
            };
            // Block 1's products run on the matrix core while the vector
            // unit forms block 0's dS; block 0's dQ products while it forms
            // block 1's.
            products(0);
            mask(0);
            products(1);
            dscores(0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * KS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                if (i < 2 * KS - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            pin(dsop[0]);  // formed here, not moved past the mask branch
            pin(dsop[1]);
            __builtin_amdgcn_sched_barrier(0);
            mask(1);
            dq_products(0);
            dq_products(1);
            dscores(1);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * D / 32; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);
                if (i < 2 * D / 32 - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            dq_products(2);
            dq_products(3);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    load_tile<D, DH, STRIDED>(Kh, N, 0, k0, ksrc, wave, kn);
    load_tile<D, DH, STRIDED>(Vh, N, 0, v0, vsrc, wave, vn);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < n_tiles; t += 2) {
        step(t, k0, v0, k1, v1);
        if (t + 1 < n_tiles) step(t + 1, k1, v1, k0, v0);
    }
    if (valid)
        store_rows<D, DH>(dQ + head_offset<DH, STRIDED>(st, bh, N, kTDQ) +
                              (size_t)qrow * row_stride<DH, STRIDED>(st, kTDQ),
                          acc, scale, g);
}

// ---------------------------------------------------------------------------
// dkdv kernel: one workgroup = 128 keys of one (batch, head); wave w owns
// keys k0 + 32w .. +31 (lane (g, j) holds key j of the wave).  Query tiles
// of 64 rows stream through LDS together with their LSE and D values.
// ---------------------------------------------------------------------------
template <typename E, int DH, bool CAUSAL, bool STRIDED>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kDkdvWaves<kLayout<DH>>, kDkdvWaves<kLayout<DH>>)))
bwd_dkdv_kernel(const E *__restrict__ Q, const E *__restrict__ K, const E *__restrict__ V,
                const E *__restrict__ dO, const float *__restrict__ LSE,
                const float *__restrict__ Delta, E *__restrict__ dK, E *__restrict__ dV, int N,
                int ntiles, float scale, float scale_log2, BwdStrides st) {
    typedef typename TileOps<E>::x8 X8;
    constexpr int D = kLayout<DH>;
    constexpr int KS = DH / 16;  // k-steps of S and dP
    __shared__ __attribute__((aligned(16))) __bf16 lds_q0[kInner * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_q1[kInner * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_o0[kInner * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_o1[kInner * D];
    // per tile: LSE (log2 units are formed on read) then D, 64 floats each
    __shared__ __attribute__((aligned(16))) float lds_s0[2 * kInner];
    __shared__ __attribute__((aligned(16))) float lds_s1[2 * kInner];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 5;
    const int j = lane & 31;

    int bh, kt;
    // Under the causal mask the first key tiles see the most queries: they
    // are issued first (no reversal).
    map_block(blockIdx.x, gridDim.x, ntiles, false, CAUSAL, 64, bh, kt);  // 2 per CU
    const int k0 = kt * kOuter;
    const E *Qh = Q + head_offset<DH, STRIDED>(st, bh, N, kTQ);
    const E *dOh = dO + head_offset<DH, STRIDED>(st, bh, N, kTDO);
    const int qn = row_stride<DH, STRIDED>(st, kTQ), don = row_stride<DH, STRIDED>(st, kTDO);
    const float *LSEh = LSE + (size_t)bh * N;
    const float *Dh = Delta + (size_t)bh * N;
    const int wk0 = k0 + wave * kRowsPerWave;
    const int key = wk0 + j;
    const bool valid = key < N;

    // K^T and V^T as B operands: lane (g, j) holds columns 16ks+8g..+7 of its key.
    const E *Kr = K + head_offset<DH, STRIDED>(st, bh, N, kTK) +
                  (size_t)key * row_stride<DH, STRIDED>(st, kTK);
    const E *Vr = V + head_offset<DH, STRIDED>(st, bh, N, kTV) +
                  (size_t)key * row_stride<DH, STRIDED>(st, kTV);
    X8 kop[KS], vop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
        if (valid) {
            const int e = 16 * ks + 8 * g;
            xk = load16(Kr + e);
            xv = load16(Vr + e);
        }
        kop[ks] = __builtin_bit_cast(X8, xk);
        vop[ks] = __builtin_bit_cast(X8, xv);
    }

    // Causal: the query tiles before the workgroup's first key see none of its keys.
    const int t_begin = CAUSAL ? k0 / kInner : 0;
    const int n_tiles = (N + kInner - 1) / kInner;

    // Q and dO may have different row strides in a strided call.
    const uint32_t qsrc = tile_src_offset<D, DH>(wave, lane, qn);
    const uint32_t dosrc = STRIDED ? tile_src_offset<D, DH>(wave, lane, don) : qsrc;
    const uint32_t rd = row_read_offset<D>(lane);
    uint32_t trd[2];
    tr_read_offsets<D>(lane, trd);

    f32x16 acck[D / 32], accv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acck[db][r] = accv[db][r] = 0.f;

    LDS3 char *const q0 = (LDS3 char *)lds_q0;
    LDS3 char *const q1 = (LDS3 char *)lds_q1;
    LDS3 char *const o0 = (LDS3 char *)lds_o0;
    LDS3 char *const o1 = (LDS3 char *)lds_o1;

    // Rows c0 .. c0+63 of Q and dO, and their LSE and D (waves 0 and 1 copy
    // those, one 4-byte direct-to-LDS load each; entries past N read as 0).
    auto load_all = [&](int c0, LDS3 char *dq_, LDS3 char *do_, LDS3 float *st) {
        load_tile<D, DH, STRIDED>(Qh, N, c0, dq_, qsrc, wave, qn);
        load_tile<D, DH, STRIDED>(dOh, N, c0, do_, dosrc, wave, don);
        if (wave < 2)
            load_vec(wave == 0 ? LSEh : Dh, N, c0, st + wave * kInner, opaque(lane));
    };

    auto step = [&](int t, const LDS3 char *qt_, const LDS3 char *ot_, const LDS3 float *st,
                    LDS3 char *nq, LDS3 char *no, LDS3 float *nst) {
        const int c0 = t * kInner;
        if (t + 1 < n_tiles) load_all(c0 + kInner, nq, no, nst);
        if constexpr (kSafeSync) {  // checking build: the copies land before any compute
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // A wave whose keys all follow this query tile has nothing to add.
        const bool active = !CAUSAL || c0 + kInner - 1 >= wk0;
        if (active) {
            // Two halves of 32 queries; element r of a half's block is query
            // c0 + 32qb + 8(r/4) + 4g + r%4 (and the lane's key).
            // S = Q K^T and dP = dO V^T of half qb.
            auto products = [&](int qb, f32x16 &s, f32x16 &dp) {
                s = f32x16{};
                dp = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const uint32_t a = row_read_at(rd, ks) + qb * 32 * D * 2;
                    const X8 qf = *reinterpret_cast<const LDS3 X8 *>(qt_ + a);
                    const X8 of = *reinterpret_cast<const LDS3 X8 *>(ot_ + a);
                    s = TileOps<E>::mfma(qf, kop[ks], s);
                    dp = TileOps<E>::mfma(of, vop[ks], dp);
                }
            };
            auto mask = [&](int qb, f32x16 &s) {
                const int qbase = c0 + 32 * qb;
                if ((CAUSAL && qbase < wk0 + kRowsPerWave - 1) || (qbase + 32 > N)) {
                    keep_branch();
                    // visible iff query >= key (causal) and query < N
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qi = qbase + 8 * (r >> 2) + 4 * g + (r & 3);
                        if (qi >= N || (CAUSAL && qi < key)) s[r] = -INFINITY;
                    }
                }
            };
            // P and dS = P o (dP - D), rounded to the element type as the B
            // operands of k-steps 2qb (queries 0-15 of the half) and 2qb + 1.
            auto scores = [&](int qb, const f32x16 &s, const f32x16 &dp, X8 *pop, X8 *dsop) {
                f32x8 plo, phi, dlo, dhi;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const f32x4 l4 = *reinterpret_cast<const LDS3 f32x4 *>(st + 32 * qb + 8 * a + 4 * g);
                    const f32x4 d4 = *reinterpret_cast<const LDS3 f32x4 *>(st + kInner + 32 * qb + 8 * a + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * a + e;
                        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -l4[e] * kLog2e));
                        const float ds = p * (dp[r] - d4[e]);
                        if (r < 8) { plo[r] = p; dlo[r] = ds; }
                        else { phi[r - 8] = p; dhi[r - 8] = ds; }
                    }
                }
                pop[0] = __builtin_convertvector(plo, X8);
                pop[1] = __builtin_convertvector(phi, X8);
                dsop[0] = __builtin_convertvector(dlo, X8);
                dsop[1] = __builtin_convertvector(dhi, X8);
            };
            // dV^T += dO^T P and dK^T += Q^T dS over the half's 32 queries.
            auto key_products = [&](int qb, const X8 *pop, const X8 *dsop) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        accv[db] = TileOps<E>::mfma(tr_read<D, X8>(ot_, trd, 2 * qb + h, db), pop[h],
                                                    accv[db]);
                        acck[db] = TileOps<E>::mfma(tr_read<D, X8>(qt_, trd, 2 * qb + h, db), dsop[h],
                                                    acck[db]);
                    }
            };
            if constexpr (D == 64) {
                // Registers allow the halves to overlap: half 1's S and dP
                // run on the matrix core while the vector unit forms half 0's
                // P and dS, and half 0's dV and dK products while it forms
                // half 1's.
                constexpr int kScoreValu = 88;  // per half: 16 x (exp, 2 fma/mul, sub, mul) + 8 cvt
                f32x16 s0, dp0, s1, dp1;
                X8 pop0[2], dsop0[2], pop1[2], dsop1[2];
                products(0, s0, dp0);
                mask(0, s0);
                products(1, s1, dp1);
                scores(0, s0, dp0, pop0, dsop0);
#pragma unroll
                for (int i = 0; i < 2 * KS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kScoreValu / (2 * KS), 0);
                }
                pin(pop0[0]);  // formed here, not moved past the mask branch
                pin(pop0[1]);
                pin(dsop0[0]);
                pin(dsop0[1]);
                __builtin_amdgcn_sched_barrier(0);
                mask(1, s1);
                key_products(0, pop0, dsop0);
                scores(1, s1, dp1, pop1, dsop1);
#pragma unroll
                for (int i = 0; i < 4 * D / 32; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kScoreValu / (4 * D / 32), 0);
                }
                pin(pop1[0]);
                pin(pop1[1]);
                pin(dsop1[0]);
                pin(dsop1[1]);
                __builtin_amdgcn_sched_barrier(0);
                key_products(1, pop1, dsop1);
            } else {
                // K, V and both accumulators take 192 registers at d = 128:
                // one half at a time, as a loop (not unrolled), which keeps
                // the halves' live ranges apart.
#pragma unroll 1
                for (int qb = 0; qb < kInner / 32; ++qb) {
                    f32x16 s = {}, dp = {};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const uint32_t a = row_read_at(rd, ks) + qb * 32 * D * 2;
                        const X8 qf = *reinterpret_cast<const LDS3 X8 *>(qt_ + a);
                        s = TileOps<E>::mfma(qf, kop[ks], s);
                        const X8 of = *reinterpret_cast<const LDS3 X8 *>(ot_ + a);
                        dp = TileOps<E>::mfma(of, vop[ks], dp);
                    }
                    mask(qb, s);
                    f32x8 plo, phi, dlo, dhi;
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const f32x4 l4 = *reinterpret_cast<const LDS3 f32x4 *>(st + 32 * qb + 8 * a + 4 * g);
                        const f32x4 d4 =
                            *reinterpret_cast<const LDS3 f32x4 *>(st + kInner + 32 * qb + 8 * a + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * a + e;
                            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -l4[e] * kLog2e));
                            const float ds = p * (dp[r] - d4[e]);
                            if (r < 8) { plo[r] = p; dlo[r] = ds; }
                            else { phi[r - 8] = p; dhi[r - 8] = ds; }
                        }
                    }
                    const X8 pop[2] = {__builtin_convertvector(plo, X8), __builtin_convertvector(phi, X8)};
                    const X8 dsop[2] = {__builtin_convertvector(dlo, X8), __builtin_convertvector(dhi, X8)};
                    key_products(qb, pop, dsop);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    LDS3 float *const s0 = (LDS3 float *)lds_s0;
    LDS3 float *const s1 = (LDS3 float *)lds_s1;
    if (t_begin < n_tiles) {
        load_all(t_begin * kInner, q0, o0, s0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int t = t_begin; t < n_tiles; t += 2) {
            step(t, q0, o0, s0, q1, o1, s1);
            if (t + 1 < n_tiles) step(t + 1, q1, o1, s1, q0, o0, s0);
        }
    }
    if (valid) {
        const int skey = opaque(key);
        store_rows<D, DH>(dK + head_offset<DH, STRIDED>(st, bh, N, kTDK) +
                              (size_t)skey * row_stride<DH, STRIDED>(st, kTDK),
                          acck, scale, g);
        store_rows<D, DH>(dV + head_offset<DH, STRIDED>(st, bh, N, kTDV) +
                              (size_t)skey * row_stride<DH, STRIDED>(st, kTDV),
                          accv, 1.f, g);
    }
}

template <typename E, int DH, bool CAUSAL, bool STRIDED>
hipError_t launch(const void *q, const void *k, const void *v, const void *o, const void *dout,
                  const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H,
                  int N, float scale, const BwdStrides &st, hipStream_t stream) {
    const int ntiles = (N + kOuter - 1) / kOuter;
    const int blocks = B * H * ntiles;
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    const E *Q = static_cast<const E *>(q), *K = static_cast<const E *>(k),
            *V = static_cast<const E *>(v), *O = static_cast<const E *>(o),
            *dO = static_cast<const E *>(dout);
    // At d = 64 the dq kernel fits three waves per SIMD (165 registers);
    // that measured 2-2.5 % faster on rows up to a few thousand keys (B4 H16
    // N2048, B16 H12 N1000, both masks) and 1.2 % slower on B1 H16 N16384
    // causal, so long rows keep two.
    bool three = false;
    if constexpr (DH == 64) {
        three = N < kDq3MaxN;
        if (three)
            hipLaunchKernelGGL((bwd_dq_kernel<E, DH, CAUSAL, STRIDED, 3>), dim3(blocks),
                               dim3(kThreads), 0, stream, Q, K, V, O, dO, lse, delta,
                               static_cast<E *>(dq), N, ntiles, scale, scale_log2, st);
    }
    if (!three)
        hipLaunchKernelGGL((bwd_dq_kernel<E, DH, CAUSAL, STRIDED>), dim3(blocks), dim3(kThreads),
                           0, stream, Q, K, V, O, dO, lse, delta, static_cast<E *>(dq), N, ntiles,
                           scale, scale_log2, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, DH, CAUSAL, STRIDED>), dim3(blocks), dim3(kThreads), 0,
                       stream, Q, K, V, dO, lse, delta, static_cast<E *>(dk),
                       static_cast<E *>(dv), N, ntiles, scale, scale_log2, st);
    return hipGetLastError();
}

template <typename E, bool STRIDED>
hipError_t launch_d(const void *q, const void *k, const void *v, const void *o, const void *dout,
                    const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H,
                    int N, int d, float scale, bool causal, const BwdStrides &st,
                    hipStream_t stream) {
#define FA_BWD_CASE(DH)                                                                          \
    case DH:                                                                                     \
        return causal ? launch<E, DH, true, STRIDED>(q, k, v, o, dout, lse, dq, dk, dv, delta, B, \
                                                     H, N, scale, st, stream)                    \
                      : launch<E, DH, false, STRIDED>(q, k, v, o, dout, lse, dq, dk, dv, delta,  \
                                                      B, H, N, scale, st, stream)
    switch (d) {
        FA_BWD_CASE(16);
        FA_BWD_CASE(32);
        FA_BWD_CASE(48);
        FA_BWD_CASE(64);
        FA_BWD_CASE(80);
        FA_BWD_CASE(96);
        FA_BWD_CASE(112);
        FA_BWD_CASE(128);
        default: return hipErrorInvalidValue;
    }
#undef FA_BWD_CASE
}

}  // namespace

hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const void *dout, const float *lse, void *dq, void *dk, void *dv,
                           float *delta, int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream) {
    const BwdStrides none = {};
    return launch_d<__bf16, false>(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale,
                                   causal, none, stream);
}

hipError_t launch_bwd_ex(bool fp16, const void *q, const void *k, const void *v, const void *o,
                         const void *dout, const float *lse, void *dq, void *dk, void *dv,
                         float *delta, int B, int H, int N, int d, float scale, bool causal,
                         const int64_t *strides, hipStream_t stream) {
    const long long hd = (long long)N * d, bd = (long long)H * hd;
    bool dense = true;
    BwdStrides st;
    for (int t = 0; t < kTensors; ++t) {
        const int64_t *x = strides + 3 * t;
        dense = dense && x[0] == bd && x[1] == hd && x[2] == d;
        st.b[t] = x[0];
        st.h[t] = x[1];
        st.n[t] = (int)x[2];
    }
    st.H = H;
    if (fp16)
        return dense ? launch_d<_Float16, false>(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N,
                                                 d, scale, causal, st, stream)
                     : launch_d<_Float16, true>(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N,
                                                d, scale, causal, st, stream);
    return dense ? launch_d<__bf16, false>(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d,
                                           scale, causal, st, stream)
                 : launch_d<__bf16, true>(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d,
                                          scale, causal, st, stream);
}

}  // namespace fa
