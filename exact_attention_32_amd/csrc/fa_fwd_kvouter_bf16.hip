// fa_fwd_kvouter_bf16.hip -- the attention forward pass in the loop order of
// Algorithm 1 of "解析 FlashAttention（2）：FlashAttention-v1 前向传播"
// (section 4): key/value blocks outside, query blocks inside, with the output
// O and the row statistics l, m kept in device memory between outer steps.
// It computes the same O and LSE as fa_fwd and exists to measure what that
// order costs: every outer step reads and writes the whole O, l, m state.
//
// Mapping onto the GPU.  The outer loop (key/value block j, 64 keys) is a
// sequence of kernel launches on one stream; the inner loop over query
// blocks i runs in parallel inside a launch, one workgroup per (batch, head,
// 128-row block i).  A workgroup of launch j does what the algorithm's inner
// body does for (i, j):
//   load K_j, V_j (direct-to-LDS) and Q_i;
//   S_ij = Q_i K_j^T (computed as S^T = K Q^T on v_mfma_f32_32x32x16_bf16);
//   block statistics: m~ = rowmax(S_ij), P~ = exp(S_ij - m~), l~ = rowsum(P~);
//   merged statistics: m_new = max(m_i, m~),
//     l_new = e^(m_i - m_new) l_i + e^(m~ - m_new) l~;
//   rescaled output: O_i <- (l_i e^(m_i - m_new) O_i + e^(m~ - m_new) P~ V_j) / l_new;
//   write O_i, l_i = l_new, m_i = m_new back.
// O_i, l_i, m_i live in an fp32 workspace (rounding O to bf16 after every
// step would add one rounding per key block).  The first step of a row block
// starts from the algorithm's initial O = 0, l = 0, m = -inf without reading
// the workspace; the last step that touches a row block writes the bf16 output and
// LSE = m*scale + ln(l) instead of the state.  Under the causal mask a
// launch j covers only the row blocks that can see a key of block j.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {
namespace {

// A head dim DH other than 64 and 128 runs in the tile layout of the next of
// the two (D): S^T takes DH/16 k-steps, the tiles and O^T have D/32
// d-blocks, and only the first DH columns of O are read, kept and stored
// (the tile columns at and past DH feed only the O^T rows past DH).
template <int DH, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
kvouter_step_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K,
                    const __bf16 *__restrict__ V, float *__restrict__ Ows,
                    float *__restrict__ Lws, float *__restrict__ Mws, __bf16 *__restrict__ O,
                    float *__restrict__ LSE, int N, int nqb, int j, int i0, float scale,
                    float scale_log2) {
    constexpr int D = DH <= 64 ? 64 : 128;
    constexpr int KS = DH / 16;
    __shared__ __attribute__((aligned(16))) __bf16 lds_k[kInner * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v[kInner * D];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 5;
    const int jq = lane & 31;
    const int per_head = nqb - i0;
    const int bh = blockIdx.x / per_head;
    const int i = i0 + blockIdx.x % per_head;
    const int r0 = i * kOuter;
    const size_t hoff = (size_t)bh * (size_t)N * DH;
    const int wrow0 = r0 + wave * kRowsPerWave;
    const int qrow = wrow0 + jq;
    const bool valid = qrow < N;
    const int c0 = j * kInner;

    // K_j, V_j to on-chip memory
    const uint32_t src = tile_src_offset<D, DH>(wave, lane);
    load_tile<D, DH>(K + hoff, N, c0, (LDS3 char *)lds_k, src, wave);
    load_tile<D, DH>(V + hoff, N, c0, (LDS3 char *)lds_v, src, wave);

    // Q_i (as the B operand of S^T = K Q^T) and the row state
    bf16x8 qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (valid) x = load16(Q + hoff + (size_t)qrow * DH + 16 * ks + 8 * g);
        qop[ks] = __builtin_bit_cast(bf16x8, x);
    }
    // The first key block a row block meets is j = 0 (every row sees key 0).
    const bool first = j == 0;
    const int last_row = min(N, r0 + kOuter) - 1;
    const int j_last = CAUSAL ? last_row / kInner : (N - 1) / kInner;
    const bool last = j == j_last;
    float m_i = -INFINITY, l_i = 0.f;
    f32x16 o_i[D / 32];
    float *orow = Ows + hoff + (size_t)qrow * DH;
    if (!first && valid) {
        m_i = Mws[(size_t)bh * N + qrow];
        l_i = Lws[(size_t)bh * N + qrow];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int col = 32 * db + 8 * a + 4 * g;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (DH == D || col < DH) x = *reinterpret_cast<const f32x4 *>(orow + col);
#pragma unroll
                for (int e = 0; e < 4; ++e) o_i[db][4 * a + e] = x[e];
            }
    } else {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o_i[db][r] = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // S^T = K_j Q_i^T (element r of s[kb] is key c0 + 32kb + 8(r/4) + 4g + r%4)
    f32x16 s[kInner / 32];
#pragma unroll
    for (int kb = 0; kb < kInner / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    const uint32_t rd = row_read_offset<D>(lane);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < kInner / 32; ++kb) {
            const bf16x8 kf = *reinterpret_cast<const LDS3 bf16x8 *>(
                (const LDS3 char *)lds_k + row_read_at(rd, ks) + kb * 32 * D * 2);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qop[ks], s[kb], 0, 0, 0);
        }
    const bool need_mask = (CAUSAL && c0 + kInner - 1 > wrow0) || (c0 + kInner > N);
    if (need_mask) {
        const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - c0 - 4 * g;
#pragma unroll
        for (int kb = 0; kb < kInner / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
    }

    // block statistics with the block's own maximum
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < kInner / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                         false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mtc = (mt == -INFINITY ? 0.f : mt) * scale_log2;
    bf16x8 pop[kInner / 16];
    float lt = 0.f;
#pragma unroll
    for (int kb = 0; kb < kInner / 32; ++kb) {
        f32x8 lo, hi;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            lo[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], scale_log2, -mtc));
            hi[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 8], scale_log2, -mtc));
            lt += lo[r] + hi[r];
        }
        pop[2 * kb] = __builtin_convertvector(lo, bf16x8);
        pop[2 * kb + 1] = __builtin_convertvector(hi, bf16x8);
    }
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt),
                                                         false, false);
        lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    // P~ V_j (O^T layout: lane (g, jq) holds query jq, d rows 32db + 8(r/4) + 4g + r%4)
    uint32_t trd[2];
    tr_read_offsets<D>(lane, trd);
    f32x16 pv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[db][r] = 0.f;
#pragma unroll
    for (int T = 0; T < kInner / 16; ++T)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            pv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                tr_read<D>((const LDS3 char *)lds_v, trd, T, db), pop[T], pv[db], 0, 0, 0);

    // merge with the stored state (a block with no visible key
    // for this row leaves it unchanged)
    const float m_new = fmaxf(m_i, mt);
    const float a_old = m_i == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_i - m_new) * scale_log2);
    const float a_blk = mt == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mt - m_new) * scale_log2);
    const float l_new = a_old * l_i + a_blk * lt;
    const float inv = 1.f / l_new;
    const float c_old = l_i * a_old * inv, c_blk = a_blk * inv;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_i[db][r] = c_old * o_i[db][r] + c_blk * pv[db][r];

    if (!valid) return;
    if (last) {
        // the algorithm's result: O and LSE = m*scale + ln(l)
        store_rows<D, DH>(O + hoff + (size_t)qrow * DH, o_i, 1.f, g);
        if (g == 0) LSE[(size_t)bh * N + qrow] = m_new * scale + logf(l_new);
    } else {
        // the state back to device memory
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int col = 32 * db + 8 * a + 4 * g;
                if (DH < D && col >= DH) continue;
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = o_i[db][4 * a + e];
                *reinterpret_cast<f32x4 *>(orow + col) = x;
            }
        if (g == 0) {
            Mws[(size_t)bh * N + qrow] = m_new;
            Lws[(size_t)bh * N + qrow] = l_new;
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                  int N, float scale, float *ows, float *lws, float *mws, hipStream_t stream) {
    const int nqb = (N + kOuter - 1) / kOuter;
    const int nkb = (N + kInner - 1) / kInner;
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    for (int j = 0; j < nkb; ++j) {
        // under the mask, row block i sees key block j iff its last row >= 64 j
        const int i0 = CAUSAL ? (j * kInner) / kOuter : 0;
        hipLaunchKernelGGL((kvouter_step_kernel<D, CAUSAL>), dim3(B * H * (nqb - i0)),
                           dim3(kThreads), 0, stream, static_cast<const __bf16 *>(q),
                           static_cast<const __bf16 *>(k), static_cast<const __bf16 *>(v), ows,
                           lws, mws, static_cast<__bf16 *>(o), lse, N, nqb, j, i0, scale,
                           scale_log2);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_kvouter_bf16(const void *q, const void *k, const void *v, void *o,
                                   float *lse, int B, int H, int N, int d, float scale,
                                   bool causal, float *ows, float *lws, float *mws,
                                   hipStream_t stream) {
#define FA_KVO_CASE(DH)                                                                          \
    case DH:                                                                                     \
        return causal ? launch<DH, true>(q, k, v, o, lse, B, H, N, scale, ows, lws, mws, stream)    \
                      : launch<DH, false>(q, k, v, o, lse, B, H, N, scale, ows, lws, mws, stream)
    switch (d) {
        FA_KVO_CASE(16);
        FA_KVO_CASE(32);
        FA_KVO_CASE(48);
        FA_KVO_CASE(64);
        FA_KVO_CASE(80);
        FA_KVO_CASE(96);
        FA_KVO_CASE(112);
        default:
            return causal ? launch<128, true>(q, k, v, o, lse, B, H, N, scale, ows, lws, mws, stream)
                          : launch<128, false>(q, k, v, o, lse, B, H, N, scale, ows, lws, mws,
                                               stream);
    }
#undef FA_KVO_CASE
}

}  // namespace fa
