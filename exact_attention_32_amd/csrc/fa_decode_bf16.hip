// fa_decode_bf16.hip -- attention of a few queries over many keys (decode)
// for gfx950: bf16 Q, K, V, O (fa_decode), or bf16 or fp16 dense tensors or
// strided views (fa_decode_ex); fp32 scores, softmax statistics and sums.
//
// What is computed: O = softmax(scale * Q K^T [+ mask]) V and the per-row
// log-sum-exp for Nq <= 16 queries over Nk keys of each (batch, head), the
// queries being the last Nq positions (under the mask query i sees keys
// j <= Nk - Nq + i; a single query sees every key, as the unit-12 causal
// lesson says of a single-token decode step).
//
// Split of the key axis (the unit-12 loop-order lesson names split-K among
// the schedules real kernels use): the Nk keys of a head are cut into S
// chunks, one single-wave workgroup per (batch, head, chunk).  Each workgroup
// produces the normalised partial output O_s and LSE_s of its chunk; a second
// kernel merges the chunks with the two-block rule of "解析 FlashAttention（2）"
// (eq. (17)/(20) for the statistics, (37) for the output):
//   LSE = ln sum_s e^(LSE_s),   O = sum_s e^(LSE_s - LSE) O_s.
// With one or two queries and few chunks (many heads, short key axes) the
// chunks of a head run as the waves of one workgroup instead and merge in
// LDS, in one launch (decode_fused_kernel).
//
// With a handful of queries the work is a matrix-vector product: about Nq
// FLOP per byte of K and V, far below the MFMA balance point, so the pass is
// bound by HBM.  One or two queries run on the vector ALUs (the split kernel
// below); from three queries on the VALU dot products no longer keep up with
// HBM and the MFMA split kernel further down takes over (measured crossover
// at B=2, H=32, Nk=8192, d=128: 49 vs 50 us at two queries, 57 vs 50 at
// three).  Layout of a wave of the VALU kernel: groups of
// G = d/8 lanes each hold one key row (16 bytes per lane), so one load
// instruction reads 64/G consecutive rows (1 KiB, coalesced); the dot product
// of a row with each query is summed over its group with DPP lane moves; every
// group runs its own online softmax (running max m, sum l, unnormalised
// output) over the rows it reads, and the groups are merged with the same
// two-block rule at the end.  K and V rows go straight from HBM into
// registers (each row is used by one wave only, so LDS would add nothing).
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include <cmath>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {
namespace {

// The two 2-byte elements of a 32-bit word (low half first), widened to fp32.
template <typename E>
__device__ __forceinline__ float elem_lo(uint32_t w);
template <typename E>
__device__ __forceinline__ float elem_hi(uint32_t w);
template <>
__device__ __forceinline__ float elem_lo<__bf16>(uint32_t w) { return __uint_as_float(w << 16); }
template <>
__device__ __forceinline__ float elem_hi<__bf16>(uint32_t w) {
    return __uint_as_float(w & 0xffff0000u);
}
template <>
__device__ __forceinline__ float elem_lo<_Float16>(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <>
__device__ __forceinline__ float elem_hi<_Float16>(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Element strides (batch, head, row) of q, k, v, o (d contiguous) for the
// STRIDED instantiations; the dense ones form bh * rows * d and d.
enum DecTensor { kDQ, kDK, kDV, kDO, kDecTensors };
struct DecStrides {
    long long b[kDecTensors], h[kDecTensors];
    int n[kDecTensors];
    int H;
};
template <int DH, bool STRIDED>
__device__ __forceinline__ size_t dec_head_offset(const DecStrides &st, int bh, int rows, int t) {
    if constexpr (STRIDED) {
        const int b = bh / st.H, h = bh - b * st.H;
        return (size_t)(b * st.b[t] + h * st.h[t]);
    } else {
        return (size_t)bh * (size_t)rows * DH;
    }
}
template <int DH, bool STRIDED>
__device__ __forceinline__ int dec_row_stride(const DecStrides &st, int t) {
    if constexpr (STRIDED) return st.n[t];
    else return DH;
}

__device__ __forceinline__ float dpp_add(float x, int ctrl_sel) {
    // ctrl values: quad_perm [1,0,3,2] = 0xb1, quad_perm [2,3,0,1] = 0x4e,
    // row_half_mirror = 0x141, row_mirror = 0x140.
    int y;
    switch (ctrl_sel) {
        case 0: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false); break;
        case 1: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false); break;
        case 2: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false); break;
        default: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false); break;
    }
    return x + __int_as_float(y);
}

// Sum over the G lanes of a group (G = 8: half a DPP row; G = 16: a row);
// every lane of the group receives the sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    x = dpp_add(x, 0);
    x = dpp_add(x, 1);
    x = dpp_add(x, 2);
    if (G == 16) x = dpp_add(x, 3);
    return x;
}

// Merge the online-softmax state (m, l, acc) of another stream into this one
// (two-block rule; m in raw score units, exponentials in base 2 with `c` =
// scale * log2(e)).  A stream that has seen no visible key has m = -inf.
template <int E>
__device__ __forceinline__ void merge_state(float &m, float &l, float *acc, float mo, float lo,
                                            const float *ao, float c) {
    const float mn = fmaxf(m, mo);
    if (mn == -INFINITY) return;
    const float a = __builtin_amdgcn_exp2f((m - mn) * c);   // 0 when m = -inf
    const float b = __builtin_amdgcn_exp2f((mo - mn) * c);
    l = l * a + lo * b;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = acc[e] * a + ao[e] * b;
    m = mn;
}

// One workgroup = one (batch*head, key chunk), with one wave per group of
// up to four queries: every wave streams the same K and V rows (the repeats
// hit the caches of the compute unit) and keeps the online-softmax state of
// its own queries only.  Writes the chunk's normalised partial output and
// LSE (0 and -inf for a query that sees no key of the chunk).
template <int NQ>
constexpr int kDecodeWaves = (NQ + 3) / 4;

// A head dim DH other than 64 and 128 runs in the layout of the next of the
// two (D): lanes whose 8 columns lie at or past DH hold zeros and load and
// store nothing; rows are DH elements apart in memory and in the partial
// outputs.
template <int DH>
constexpr int kDecLayout = DH <= 64 ? 64 : 128;

// The online-softmax state of one wave over keys [k0, k1) of head bh for
// queries qbase .. qbase + NQW - 1 (NQW = min(NQ, 4)), merged over the
// wave's RPW row groups: on return every lane holds its group's columns
// col*8 .. +7 of the state (m, l, unnormalised acc), identical in all groups.
template <typename E, int DH, int NQ, bool CAUSAL, bool STRIDED>
__device__ __forceinline__ void chunk_state(const E *__restrict__ Q, const E *__restrict__ K,
                                            const E *__restrict__ V, int Nq, int Nk, int bh,
                                            int k0, int k1, int qbase, float scale_log2,
                                            const DecStrides &st, float (&m)[NQ < 4 ? NQ : 4],
                                            float (&l)[NQ < 4 ? NQ : 4],
                                            float (&acc)[NQ < 4 ? NQ : 4][8]) {
    constexpr int D = kDecLayout<DH>;
    constexpr int G = D / 8;       // lanes per key row
    constexpr int RPW = 64 / G;    // rows per load instruction
    constexpr int NQW = NQ < 4 ? NQ : 4;  // queries per wave
    constexpr int ROUNDS = NQW <= 2 ? 8 : 4;
    constexpr int BLK = RPW * ROUNDS;  // keys per block of loads

    const int lane = threadIdx.x & 63;
    const int grp = lane / G;
    const int col = lane % G;
    const bool has_cols = DH == D || col * 8 < DH;  // this lane's columns exist

    // This lane's 8 columns of every query of the wave, widened to fp32.
    float qf[NQW][8];
#pragma unroll
    for (int qi = 0; qi < NQW; ++qi) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qbase + qi < Nq && has_cols)
            w = *reinterpret_cast<const u32x4 *>(
                Q + dec_head_offset<DH, STRIDED>(st, bh, Nq, kDQ) +
                (size_t)(qbase + qi) * dec_row_stride<DH, STRIDED>(st, kDQ) + col * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[qi][2 * e] = elem_lo<E>(w[e]);
            qf[qi][2 * e + 1] = elem_hi<E>(w[e]);
        }
    }
#pragma unroll
    for (int qi = 0; qi < NQW; ++qi) {
        m[qi] = -INFINITY;
        l[qi] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qi][e] = 0.f;
    }

    const E *Kh = K + dec_head_offset<DH, STRIDED>(st, bh, Nk, kDK) + col * 8;
    const E *Vh = V + dec_head_offset<DH, STRIDED>(st, bh, Nk, kDV) + col * 8;
    const int kn = dec_row_stride<DH, STRIDED>(st, kDK), vn = dec_row_stride<DH, STRIDED>(st, kDV);
    for (int base = k0; base < k1; base += BLK) {
        u32x4 kr[ROUNDS], vr[ROUNDS];
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const int j = base + r * RPW + grp;
            kr[r] = vr[r] = u32x4{0u, 0u, 0u, 0u};
            if (j < k1 && has_cols) {
                kr[r] = *reinterpret_cast<const u32x4 *>(Kh + (size_t)j * kn);
                vr[r] = *reinterpret_cast<const u32x4 *>(Vh + (size_t)j * vn);
            }
        }
        // Scores of the block's rows (identical in all G lanes of a group).
        float sc[ROUNDS][NQW];
#pragma unroll
        for (int r = 0; r < ROUNDS; ++r) {
            const int j = base + r * RPW + grp;
#pragma unroll
            for (int qi = 0; qi < NQW; ++qi) {
                float x = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x = __builtin_fmaf(qf[qi][2 * e], elem_lo<E>(kr[r][e]), x);
                    x = __builtin_fmaf(qf[qi][2 * e + 1], elem_hi<E>(kr[r][e]), x);
                }
                x = group_sum<G>(x);
                const bool hidden = j >= k1 || (CAUSAL && j > Nk - Nq + qbase + qi);
                sc[r][qi] = hidden ? -INFINITY : x;
            }
        }
        // Online softmax of this group's stream, one update per block.
#pragma unroll
        for (int qi = 0; qi < NQW; ++qi) {
            float mb = sc[0][qi];
#pragma unroll
            for (int r = 1; r < ROUNDS; ++r) mb = fmaxf(mb, sc[r][qi]);
            const float mn = fmaxf(m[qi], mb);
            if (mn == -INFINITY) continue;  // nothing visible yet
            const float alpha = __builtin_amdgcn_exp2f((m[qi] - mn) * scale_log2);
            const float mc = mn * scale_log2;
            float ps = 0.f, add[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) add[e] = 0.f;
#pragma unroll
            for (int r = 0; r < ROUNDS; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r][qi], scale_log2, -mc));
                ps += p;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    add[2 * e] = __builtin_fmaf(p, elem_lo<E>(vr[r][e]), add[2 * e]);
                    add[2 * e + 1] = __builtin_fmaf(p, elem_hi<E>(vr[r][e]), add[2 * e + 1]);
                }
            }
            l[qi] = l[qi] * alpha + ps;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[qi][e] = acc[qi][e] * alpha + add[e];
            m[qi] = mn;
        }
    }

    // Merge the RPW group streams of the wave (lanes G, 2G, ... apart).
#pragma unroll
    for (int qi = 0; qi < NQW; ++qi) {
#pragma unroll
        for (int off = G; off < 64; off <<= 1) {
            const float mo = __shfl_xor(m[qi], off);
            const float lo = __shfl_xor(l[qi], off);
            float ao[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ao[e] = __shfl_xor(acc[qi][e], off);
            merge_state<8>(m[qi], l[qi], acc[qi], mo, lo, ao, scale_log2);
        }
    }

}

template <typename E, int DH, int NQ, bool CAUSAL, bool STRIDED>
__global__ void __launch_bounds__(64 * kDecodeWaves<NQ>)
decode_split_kernel(const E *__restrict__ Q, const E *__restrict__ K, const E *__restrict__ V,
                    float *__restrict__ o_part, float *__restrict__ lse_part, int Nq, int Nk,
                    int S, int chunk, float scale, float scale_log2, DecStrides st) {
    constexpr int D = kDecLayout<DH>;
    constexpr int G = D / 8;              // lanes per key row
    constexpr int NQW = NQ < 4 ? NQ : 4;  // queries per wave

    const int lane = threadIdx.x & 63;
    const int qbase = NQW * (threadIdx.x >> 6);  // first query of this wave
    const int grp = lane / G;
    const int col = lane % G;
    const int s = blockIdx.x % S;
    const int bh = blockIdx.x / S;
    const int k0 = s * chunk;
    const int k1 = min(Nk, k0 + chunk);
    const bool has_cols = DH == D || col * 8 < DH;  // this lane's columns exist
    float m[NQW], l[NQW], acc[NQW][8];
    chunk_state<E, DH, NQ, CAUSAL, STRIDED>(Q, K, V, Nq, Nk, bh, k0, k1, qbase, scale_log2, st, m, l,
                                            acc);

    if (grp == 0) {
#pragma unroll
        for (int qi = 0; qi < NQW; ++qi) {
            if (qbase + qi >= Nq) break;
            const size_t prow = ((size_t)bh * S + s) * Nq + qbase + qi;
            const float inv = l[qi] > 0.f ? 1.f / l[qi] : 0.f;
            float *dst = o_part + prow * DH + col * 8;
            if (has_cols) {
#pragma unroll
                for (int e = 0; e < 8; e += 4)
                    *reinterpret_cast<float4 *>(dst + e) =
                        make_float4(acc[qi][e] * inv, acc[qi][e + 1] * inv, acc[qi][e + 2] * inv,
                                    acc[qi][e + 3] * inv);
            }
            if (col == 0) lse_part[prow] = l[qi] > 0.f ? m[qi] * scale + logf(l[qi]) : -INFINITY;
        }
    }
}

// Split and merge in one launch, for one or two queries and at most
// kFusedMaxChunks chunks: one workgroup per (batch, head) with one wave per
// chunk.  Every wave leaves its chunk's unnormalised state (m, l, acc) in LDS,
// and after a barrier the workgroup merges the S states with the same
// two-block rule, O = sum_s 2^((m_s - M) c) acc_s / L with M = max_s m_s and
// L = sum_s 2^((m_s - M) c) l_s, LSE = M scale + ln L (c = scale log2 e).  A
// chunk in which a query sees no key has m = -inf and adds nothing; every
// query sees at least one key (Nk >= Nq), so M is finite.  Saves the second
// launch and the round trip of the partials through HBM where the heads are
// many and the chunks few.
template <int NQ>
constexpr int kFusedMaxChunks = NQ == 1 ? 16 : 8;  // (register budget of the waves)

template <typename E, int DH, int NQ, bool CAUSAL, bool STRIDED>
__global__ void __launch_bounds__(64 * kFusedMaxChunks<NQ>)
decode_fused_kernel(const E *__restrict__ Q, const E *__restrict__ K, const E *__restrict__ V,
                    E *__restrict__ O, float *__restrict__ LSE, int Nq, int Nk, int chunk,
                    float scale, float scale_log2, DecStrides st) {
    static_assert(NQ <= 2, "one wave per chunk holds all queries");
    constexpr int D = kDecLayout<DH>;
    constexpr int G = D / 8;
    __shared__ float sm_acc[kFusedMaxChunks<NQ>][NQ][DH];
    __shared__ float sm_m[kFusedMaxChunks<NQ>][NQ], sm_l[kFusedMaxChunks<NQ>][NQ];

    const int lane = threadIdx.x & 63;
    const int s = threadIdx.x >> 6;  // chunk of this wave
    const int S = blockDim.x >> 6;
    const int bh = blockIdx.x;
    const int grp = lane / G;
    const int col = lane % G;
    const int k0 = s * chunk;
    const int k1 = min(Nk, k0 + chunk);
    float m[NQ], l[NQ], acc[NQ][8];
    chunk_state<E, DH, NQ, CAUSAL, STRIDED>(Q, K, V, Nq, Nk, bh, k0, k1, 0, scale_log2, st, m, l,
                                            acc);
    if (grp == 0) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if (qi >= Nq) break;
            if (DH == D || col * 8 < DH) {
#pragma unroll
                for (int e = 0; e < 8; e += 4)
                    *reinterpret_cast<float4 *>(&sm_acc[s][qi][col * 8 + e]) =
                        make_float4(acc[qi][e], acc[qi][e + 1], acc[qi][e + 2], acc[qi][e + 3]);
            }
            if (col == 0) {
                sm_m[s][qi] = m[qi];
                sm_l[s][qi] = l[qi];
            }
        }
    }
    __syncthreads();

    for (int t = threadIdx.x; t < Nq * DH; t += blockDim.x) {
        const int qi = t / DH, c = t - qi * DH;
        float mx = sm_m[0][qi];
        for (int u = 1; u < S; ++u) mx = fmaxf(mx, sm_m[u][qi]);
        float lsum = 0.f, o = 0.f;
        for (int u = 0; u < S; ++u) {
            const float w = __builtin_amdgcn_exp2f((sm_m[u][qi] - mx) * scale_log2);
            lsum = __builtin_fmaf(w, sm_l[u][qi], lsum);
            o = __builtin_fmaf(w, sm_acc[u][qi][c], o);
        }
        O[dec_head_offset<DH, STRIDED>(st, bh, Nq, kDO) +
          (size_t)qi * dec_row_stride<DH, STRIDED>(st, kDO) + c] = (E)(o / lsum);
        if (c == 0) LSE[(size_t)bh * Nq + qi] = mx * scale + logf(lsum);
    }
}

// ---------------------------------------------------------------------------
// MFMA split kernel, for more than kDecodeValuQueries queries.  The VALU
// kernel above spends Nq DPP-reduced dot products per key row and stops
// being bound by HBM at three queries; with the queries as one
// 32-column block (columns past Nq are zero) the two products are MFMA
// work, as in the forward kernels: S^T = K Q^T with K tiles read row-wise
// from LDS, O^T += V^T P^T with V tiles read through the LDS transpose read,
// the softmax in between (lazy exponent base, as in the forward pass).  Its
// cost no longer grows with Nq.
//
// One wave per (batch*head, key chunk).  The chunk's keys go through 32-key
// tiles of K and V copied global -> LDS by direct-to-LDS buffer loads into
// three buffers private to the wave, two tiles ahead of the one being
// multiplied; the wave waits for its own copies by vmcnt (no barrier), and
// for its own reads of a buffer (lgkmcnt) before refilling it.  LDS layout
// and read offsets: the shared swizzle of fa_tiles.h (conflict-free for
// both read patterns).
constexpr int kDecTile = 32;  // keys per LDS tile
// Largest half-row probability sum accepted against the current exponent
// base (every probability of the tile is then at most this): 2^32 for bf16
// probabilities, 2^15 for fp16 ones (largest finite value 65504).
template <typename E>
constexpr float kDecSumMax = 4294967296.f;
template <>
constexpr float kDecSumMax<_Float16> = 32768.f;

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]); a counter not waited for is set to its maximum.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Copy of the 32-key tile of K and V starting at key c0 (keys at or past
// k1 read as zeros) into kd and vd: load u of the wave writes LDS bytes
// u*1024 + 16*lane and fetches the global offset src[u] (row and swizzled
// chunk).  (A function of its own: a buffer descriptor local to a lambda
// makes the host pass drop the kernel's launch stub.)
template <int DH, int kLoads, bool STRIDED>
__device__ __forceinline__ void decode_copy_tile(const void *Kh, const void *Vh, int c0, int k1,
                                                 LDS3 char *kd, LDS3 char *vd,
                                                 const uint32_t *ksrc, const uint32_t *vsrc,
                                                 int kn, int vn) {
    const uint32_t rows = (uint32_t)max(0, min(kDecTile, k1 - c0));
    const uint32_t kbytes = __builtin_amdgcn_readfirstlane(
        STRIDED ? (rows ? (rows - 1) * (uint32_t)kn * 2u + DH * 2u : 0u) : rows * (uint32_t)(DH * 2));
    const uint32_t vbytes = __builtin_amdgcn_readfirstlane(
        STRIDED ? (rows ? (rows - 1) * (uint32_t)vn * 2u + DH * 2u : 0u) : rows * (uint32_t)(DH * 2));
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc((const char *)Kh + (size_t)c0 * (size_t)kn * 2, kbytes);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc((const char *)Vh + (size_t)c0 * (size_t)vn * 2, vbytes);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS3 void *)(kd + u * 1024), 16, ksrc[u], 0,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS3 void *)(vd + u * 1024), 16, vsrc[u], 0,
                                                 0, 0);
    }
}

// (Two waves per SIMD at d = 64 keep the accumulators in VGPRs; at d = 128
// the three tiles of LDS allow one workgroup per SIMD, and the compiler then
// keeps them in AGPRs, costing only VALU slots this HBM-bound kernel has
// spare.)
// A head dim DH other than 64 and 128 runs in the tile layout of the next of
// the two (D): S^T takes DH/16 k-steps, O^T has D/32 d-blocks, the tile rows
// are gathered at the DH row stride (the columns at and past DH hold the
// next row's leading elements, or zeros past the tile, and feed only the
// O^T rows at and past DH), and the first DH columns are stored.
template <typename E, int DH, bool CAUSAL, bool STRIDED>
__global__ void __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(kDecLayout<DH> == 64 ? 2 : 1)))
decode_mfma_kernel(const E *__restrict__ Q, const E *__restrict__ K, const E *__restrict__ V,
                   float *__restrict__ o_part, float *__restrict__ lse_part, int Nq, int Nk,
                   int S, int chunk, float scale, float scale_log2, DecStrides st) {
    typedef typename TileOps<E>::x8 X8;
    constexpr int D = kDecLayout<DH>;
    constexpr int KS = DH / 16;                // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;                 // 32-wide d blocks of O^T
    constexpr int kRowsPerLoad = 64 / (D / 8);  // rows per 1 KiB load (4 or 8)
    constexpr int kLoads = kDecTile / kRowsPerLoad;  // per operand and tile
    constexpr int kTileBytes = kDecTile * D * 2;
    __shared__ __attribute__((aligned(16))) __bf16 lk0[kDecTile * D];
    __shared__ __attribute__((aligned(16))) __bf16 lk1[kDecTile * D];
    __shared__ __attribute__((aligned(16))) __bf16 lk2[kDecTile * D];
    __shared__ __attribute__((aligned(16))) __bf16 lv0[kDecTile * D];
    __shared__ __attribute__((aligned(16))) __bf16 lv1[kDecTile * D];
    __shared__ __attribute__((aligned(16))) __bf16 lv2[kDecTile * D];

    const int lane = threadIdx.x;
    const int g = lane >> 5;
    const int j = lane & 31;  // query column of this lane
    const int s = blockIdx.x % S;
    const int bh = blockIdx.x / S;
    const int k0 = s * chunk;
    const int k1 = min(Nk, k0 + chunk);
    const int n_tiles = (k1 - k0 + kDecTile - 1) / kDecTile;

    // Q^T as the B operand: lane (g, j) holds query j (zero past Nq),
    // columns 16ks + 8g .. +7.
    X8 qop[KS];
    const E *Qr = Q + dec_head_offset<DH, STRIDED>(st, bh, Nq, kDQ) +
                  (size_t)j * dec_row_stride<DH, STRIDED>(st, kDQ);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (j < Nq) x = load16(Qr + 16 * ks + 8 * g);
        qop[ks] = __builtin_bit_cast(X8, x);
    }
    // Query j sees keys up to vis (below the chunk's end; under the mask,
    // keys <= Nk - Nq + j).
    const int vis = CAUSAL ? min(k1 - 1, Nk - Nq + j) : k1 - 1;
    const int vis_lo = CAUSAL ? min(k1 - 1, Nk - Nq) : k1 - 1;  // the least of the wave's

    // Tile copies: load u fills LDS chunk positions u*64 + lane, i.e. row
    // u*kRowsPerLoad + lane / (D/8), stored chunk lane % (D/8), and fetches the
    // logical chunk the swizzle stores there.
    // A position whose logical chunk lies at or past DH/8 fetches chunk
    // c mod DH/8 of the same row (every byte read belongs to a row).
    const int kn = dec_row_stride<DH, STRIDED>(st, kDK), vn = dec_row_stride<DH, STRIDED>(st, kDV);
    uint32_t ksrc[kLoads], vsrc[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int r = u * kRowsPerLoad + lane / (D / 8);
        const int p = lane % (D / 8);
        int c = p ^ swz<D>(r);
        if (DH < D) c %= DH / 8;
        ksrc[u] = (uint32_t)(r * kn * 2 + (c << 4));
        vsrc[u] = STRIDED ? (uint32_t)(r * vn * 2 + (c << 4)) : ksrc[u];
    }
    const E *Kh = K + dec_head_offset<DH, STRIDED>(st, bh, Nk, kDK);
    const E *Vh = V + dec_head_offset<DH, STRIDED>(st, bh, Nk, kDV);
    auto copy_tile = [&](int t, LDS3 char *kd, LDS3 char *vd) __attribute__((always_inline)) {
        decode_copy_tile<DH, kLoads, STRIDED>(Kh, Vh, k0 + t * kDecTile, k1, kd, vd, ksrc, vsrc,
                                              kn, vn);
    };
    static_assert(kLoads * 1024 == kTileBytes, "tile copy");

    const uint32_t rd = row_read_offset<D>(lane);
    uint32_t trd[2];
    tr_read_offsets<D>(lane, trd);

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m_run = -INFINITY, mc_run = -INFINITY, l_run = 0.f;
    // Sum of the rounded probabilities that multiply V (the partial output is
    // normalised by it; the partial LSE uses the fp32 sum l).
    float lr_run = 0.f;
    const X8 sel = rowsum_selector<E>(lane);

    // Probabilities of the tile's 32 keys against base mcx (scaled log2
    // units) as P^T operands (keys 0-15, 16-31), and their half-wave sum.
    auto exps = [&](const f32x16 &sc, float mcx, X8 (&p)[2]) __attribute__((always_inline)) {
        f32x8 lo, hi;
        float ra = 0.f, rb = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            lo[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], scale_log2, -mcx));
            hi[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r + 8], scale_log2, -mcx));
            ra += lo[r];
            rb += hi[r];
        }
        p[0] = __builtin_convertvector(lo, X8);
        p[1] = __builtin_convertvector(hi, X8);
        return ra + rb;
    };

    // One tile: S^T, mask, softmax (lazy base: the base moves to the row
    // maximum only when a half-row sum leaves (0, 2^32] or is not finite),
    // O^T += V^T P^T; then the buffers are refilled with tile t + 3.
    auto tile = [&](int t, LDS3 char *kt, LDS3 char *vt) __attribute__((always_inline)) {
        // this tile's copies are the oldest outstanding ones
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * kLoads));
        f32x16 sc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const X8 kf = *reinterpret_cast<const LDS3 X8 *>(kt + row_read_at(rd, ks));
            sc = TileOps<E>::mfma(kf, qop[ks], sc);
        }
        // Element r of sc is key c0 + 8(r/4) + 4g + r%4 of query j.
        const int c0 = k0 + t * kDecTile;
        if (c0 + kDecTile - 1 > vis_lo) {
            const int lim = vis - c0 - 4 * g;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) > lim) sc[r] = -INFINITY;
        }
        X8 pp[2];
        float rs = exps(sc, mc_run, pp);
        if (__ballot(!(rs <= kDecSumMax<E>))) {
            float mt = sc[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt),
                                                                 __float_as_uint(mt), false, false);
                mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float m_new = fmaxf(m_run, mt);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha =
                (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
            mc_run = m_use * scale_log2;
            m_run = m_use;
            l_run *= alpha;
            lr_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            rs = exps(sc, mc_run, pp);
        }
        l_run += rs;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                acc[db] = TileOps<E>::mfma(tr_read<D, X8>(vt, trd, tt, db), pp[tt], acc[db]);
        f32x4 lt = {0.f, 0.f, 0.f, 0.f};
        lt = TileOps<E>::mfma16(sel, pp[0], lt);
        lt = TileOps<E>::mfma16(sel, pp[1], lt);
        lr_run += lt[0];
        // every read of these buffers has completed before they are refilled
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        copy_tile(t + 3, kt, vt);
        if constexpr (kSafeSync) __builtin_amdgcn_s_waitcnt(0);  // checking build
    };

    LDS3 char *const kb0 = (LDS3 char *)lk0;
    LDS3 char *const kb1 = (LDS3 char *)lk1;
    LDS3 char *const kb2 = (LDS3 char *)lk2;
    LDS3 char *const vb0 = (LDS3 char *)lv0;
    LDS3 char *const vb1 = (LDS3 char *)lv1;
    LDS3 char *const vb2 = (LDS3 char *)lv2;
    copy_tile(0, kb0, vb0);
    copy_tile(1, kb1, vb1);
    copy_tile(2, kb2, vb2);
    // Whole rounds of three tiles (tiles past the chunk are empty copies and
    // fully masked): every round issues the same copies in the same order,
    // so the waits on the copies can be counted exactly.
    for (int t = 0; t < n_tiles; t += 3) {
        tile(t, kb0, vb0);
        tile(t + 1, kb1, vb1);
        tile(t + 2, kb2, vb2);
    }
    // No copy is left in flight when the wave ends.
    __builtin_amdgcn_s_waitcnt(0);

    float l_tot;
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                         __float_as_uint(l_run), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (j < Nq) {
        const size_t prow = ((size_t)bh * S + s) * Nq + j;
        const float inv = lr_run > 0.f ? 1.f / lr_run : 0.f;
        float *dst = o_part + prow * DH;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int col = 32 * db + 8 * a + 4 * g;
                if (DH < D && col >= DH) continue;
                *reinterpret_cast<float4 *>(dst + col) =
                    make_float4(acc[db][4 * a] * inv, acc[db][4 * a + 1] * inv,
                                acc[db][4 * a + 2] * inv, acc[db][4 * a + 3] * inv);
            }
        if (g == 0) lse_part[prow] = l_tot > 0.f ? m_run * scale + logf(l_tot) : -INFINITY;
    }
}

// Merge kernel: one workgroup of 256 threads per output row (batch*head,
// query) combines the row's S partial rows.  Every query sees key 0, so some
// chunk has a finite LSE.
//  1. LSE = ln sum_s e^(LSE_s): each thread folds its share of the S values
//     into a (max, sum) pair; the pairs are merged across the workgroup.
//  2. O = sum_s e^(LSE_s - LSE) O_s: the weights of up to kMergeChunk chunks
//     at a time go to LDS; thread t adds column t % D of the chunks
//     s = t / D (mod 256 / D), eight loads in flight per thread; the 256 / D slices
//     are summed through LDS at the end.
constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 1024;

__device__ __forceinline__ void fold_lse(float &m, float &l, float x) {
    if (x == -INFINITY) return;
    if (x > m) {
        l = l * __builtin_amdgcn_exp2f((m - x) * kLog2e) + 1.f;
        m = x;
    } else {
        l += __builtin_amdgcn_exp2f((x - m) * kLog2e);
    }
}

__device__ __forceinline__ void merge_pair(float &m, float &l, float mo, float lo) {
    const float mn = fmaxf(m, mo);
    if (mn == -INFINITY) return;
    l = l * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + lo * __builtin_amdgcn_exp2f((mo - mn) * kLog2e);
    m = mn;
}

template <typename E, int DH, bool STRIDED>
__global__ void __launch_bounds__(kMergeThreads)
decode_merge_kernel(const float *__restrict__ o_part, const float *__restrict__ lse_part,
                    E *__restrict__ O, float *__restrict__ LSE, int Nq, int S, DecStrides st) {
    // Threads are laid out over D >= DH columns (a divisor of the workgroup
    // size); those of the columns at and past DH add nothing.
    constexpr int D = DH <= 64 ? 64 : 128;
    constexpr int kSlices = kMergeThreads / D;
    __shared__ float wts[kMergeChunk];
    __shared__ float red_m[kMergeThreads / 64], red_l[kMergeThreads / 64];
    __shared__ float part[kMergeThreads];
    const int row = blockIdx.x;  // bh * Nq + qi
    const int bh = row / Nq, qi = row - bh * Nq;
    const int t = threadIdx.x;
    const float *lp = lse_part + (size_t)bh * S * Nq + qi;

    float m = -INFINITY, l = 0.f;
    for (int s = t; s < S; s += kMergeThreads) fold_lse(m, l, lp[(size_t)s * Nq]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) merge_pair(m, l, __shfl_xor(m, off), __shfl_xor(l, off));
    if ((t & 63) == 0) {
        red_m[t >> 6] = m;
        red_l[t >> 6] = l;
    }
    __syncthreads();
    m = red_m[0];
    l = red_l[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) merge_pair(m, l, red_m[w], red_l[w]);
    const float lse = m + logf(l);

    const int c = t % D, slice = t / D;
    // Eight independent partial sums per thread, so that eight loads of
    // partial rows are in flight at once (the loop is bound by their latency).
    constexpr int kAcc = 8;
    float acc[kAcc];
#pragma unroll
    for (int u = 0; u < kAcc; ++u) acc[u] = 0.f;
    for (int s0 = 0; s0 < S; s0 += kMergeChunk) {
        const int n = min(kMergeChunk, S - s0);
        __syncthreads();  // the previous chunk's weights are no longer read
        for (int s = t; s < n; s += kMergeThreads)
            wts[s] = __builtin_amdgcn_exp2f((lp[(size_t)(s0 + s) * Nq] - lse) * kLog2e);
        __syncthreads();
        const float *op = o_part + (((size_t)bh * S + s0) * Nq + qi) * DH + c;
        const size_t stride = (size_t)Nq * DH;
        int s = c < DH ? slice : n;
        for (; s + (kAcc - 1) * kSlices < n; s += kAcc * kSlices) {
#pragma unroll
            for (int u = 0; u < kAcc; ++u)
                acc[u] = __builtin_fmaf(wts[s + u * kSlices], op[(size_t)(s + u * kSlices) * stride],
                                        acc[u]);
        }
        for (; s < n; s += kSlices) acc[0] = __builtin_fmaf(wts[s], op[(size_t)s * stride], acc[0]);
    }
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < kAcc; ++u) sum += acc[u];
    part[t] = sum;
    __syncthreads();
    if (slice == 0 && c < DH) {
        float o = part[c];
#pragma unroll
        for (int k = 1; k < kSlices; ++k) o += part[k * D + c];
        O[dec_head_offset<DH, STRIDED>(st, bh, Nq, kDO) +
          (size_t)qi * dec_row_stride<DH, STRIDED>(st, kDO) + c] = (E)o;
        if (c == 0) LSE[row] = lse;
    }
}

template <typename E, int DH, int NQ, bool CAUSAL, bool STRIDED>
hipError_t launch_nq(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                     int H, int Nq, int Nk, int S, int chunk, float scale, float *o_part,
                     float *lse_part, const DecStrides &st, hipStream_t stream) {
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    const E *Q = static_cast<const E *>(q), *K = static_cast<const E *>(k),
            *V = static_cast<const E *>(v);
    if constexpr (NQ <= kDecodeValuQueries) {
        if (S <= kFusedMaxChunks<NQ>) {
            hipLaunchKernelGGL((decode_fused_kernel<E, DH, NQ, CAUSAL, STRIDED>), dim3(B * H),
                               dim3(64 * S), 0, stream, Q, K, V, static_cast<E *>(o), lse, Nq, Nk,
                               chunk, scale, scale_log2, st);
            return hipGetLastError();
        }
    }
    if constexpr (NQ > kDecodeValuQueries)
        hipLaunchKernelGGL((decode_mfma_kernel<E, DH, CAUSAL, STRIDED>), dim3(B * H * S), dim3(64),
                           0, stream, Q, K, V, o_part, lse_part, Nq, Nk, S, chunk, scale,
                           scale_log2, st);
    else
        hipLaunchKernelGGL((decode_split_kernel<E, DH, NQ, CAUSAL, STRIDED>), dim3(B * H * S),
                           dim3(64 * kDecodeWaves<NQ>), 0, stream, Q, K, V, o_part, lse_part, Nq,
                           Nk, S, chunk, scale, scale_log2, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<E, DH, STRIDED>), dim3(B * H * Nq),
                       dim3(kMergeThreads), 0, stream, o_part, lse_part, static_cast<E *>(o), lse,
                       Nq, S, st);
    return hipGetLastError();
}

template <typename E, int DH, bool CAUSAL, bool STRIDED>
hipError_t launch_q(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int H, int Nq, int Nk, int S, int chunk, float scale, float *o_part,
                    float *lse_part, const DecStrides &st, hipStream_t stream) {
#define FA_DECODE_NQ(NQ)                                                                        \
    return launch_nq<E, DH, NQ, CAUSAL, STRIDED>(q, k, v, o, lse, B, H, Nq, Nk, S, chunk, scale, \
                                                 o_part, lse_part, st, stream)
    if (Nq <= 1) FA_DECODE_NQ(1);
    if (Nq <= 2) FA_DECODE_NQ(2);
    // From three queries on the MFMA kernel runs, whatever the count.
    FA_DECODE_NQ(16);
#undef FA_DECODE_NQ
}

template <typename E, bool STRIDED>
hipError_t launch_e(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int H, int Nq, int Nk, int d, float scale, bool causal, int S, float *o_part,
                    float *lse_part, const DecStrides &st, hipStream_t stream) {
    // The MFMA kernel walks its chunk in rounds of three 32-key tiles, so its
    // chunks are whole rounds (a chunk of 256 keys would run 9 tile slots for
    // 8 tiles); the vector-ALU kernels take whole 64-key blocks.
    const int chunk = decode_chunk(Nk, S, Nq > kDecodeValuQueries ? 3 * kDecTile : 64);
    S = (Nk + chunk - 1) / chunk;  // no empty chunk
#define FA_DEC_CASE(DH)                                                                         \
    case DH:                                                                                    \
        return causal ? launch_q<E, DH, true, STRIDED>(q, k, v, o, lse, B, H, Nq, Nk, S, chunk, \
                                                       scale, o_part, lse_part, st, stream)    \
                      : launch_q<E, DH, false, STRIDED>(q, k, v, o, lse, B, H, Nq, Nk, S,       \
                                                        chunk, scale, o_part, lse_part, st,     \
                                                        stream)
    switch (d) {
        FA_DEC_CASE(16);
        FA_DEC_CASE(32);
        FA_DEC_CASE(48);
        FA_DEC_CASE(64);
        FA_DEC_CASE(80);
        FA_DEC_CASE(96);
        FA_DEC_CASE(112);
        FA_DEC_CASE(128);
        default: return hipErrorInvalidValue;
    }
#undef FA_DEC_CASE
}

}  // namespace

// Fixed scratch of the allocation-free decode entry point (fa_decode_noalloc):
// the split kernel's fp32 partials live here instead of in a caller workspace.
// Each device holds its own copy for the life of the process; host code must
// use the device address from hipGetSymbolAddress, never this name.
static __device__ __align__(256) unsigned char decode_scratch_mem[kDecodeScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(decode_scratch_mem));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_decode_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                              int B, int H, int Nq, int Nk, int d, float scale, bool causal,
                              int S, float *o_part, float *lse_part, hipStream_t stream) {
    const DecStrides none = {};
    return launch_e<__bf16, false>(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, S, o_part,
                                   lse_part, none, stream);
}

hipError_t launch_decode_ex(bool fp16, const void *q, const void *k, const void *v, void *o,
                            float *lse, int B, int H, int Nq, int Nk, int d, float scale,
                            bool causal, int S, float *o_part, float *lse_part,
                            const int64_t *strides, hipStream_t stream) {
    DecStrides st;
    bool dense = true;
    for (int t = 0; t < kDecTensors; ++t) {
        const int64_t *x = strides + 3 * t;
        const long long rows = (t == kDQ || t == kDO) ? Nq : Nk;
        dense = dense && x[0] == (long long)H * rows * d && x[1] == rows * d && x[2] == d;
        st.b[t] = x[0];
        st.h[t] = x[1];
        st.n[t] = (int)x[2];
    }
    st.H = H;
    if (fp16)
        return dense ? launch_e<_Float16, false>(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, S,
                                                 o_part, lse_part, st, stream)
                     : launch_e<_Float16, true>(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, S,
                                                o_part, lse_part, st, stream);
    return dense ? launch_e<__bf16, false>(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, S,
                                           o_part, lse_part, st, stream)
                 : launch_e<__bf16, true>(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, S,
                                          o_part, lse_part, st, stream);
}

}  // namespace fa
