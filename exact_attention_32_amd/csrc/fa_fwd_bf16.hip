// fa_fwd_bf16.hip -- fused attention forward for gfx950: bf16 tensors (the
// fa_fwd path) and, through the same template, fp16 tensors and strided
// views (fa_fwd_ex); head dims 16, 32, ..., 128 (multiples of 16); fp32
// scores, softmax statistics and accumulator.
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
// Two kernels share the operand layouts, LDS swizzles, softmax and grid
// mapping described here: fwd_kernel (every head dim but 128, except causal
// d = 64 on long rows) and fwd_pipe_kernel (head dim 128 with 8-wave
// workgroups; causal d = 64 with N >= 8192 with 4-wave ones), which reorders
// the work inside a wave into a software pipeline; see its own comment
// further down.
//
// Mapping onto CDNA4 (described for fwd_kernel at d = 128; d/16 k-steps and
// d/32 output blocks otherwise, with the LDS layouts given at k_swz / v_swz
// below)
// ------------------
// * One workgroup = 4 wavefronts = 128 query rows of one (batch, head); each
//   wave owns 32 rows for the whole key loop (Q, the output accumulator and
//   the running max / sum never leave registers).  Two workgroups (three
//   at d <= 64, where a wave needs at most 168 registers) share a compute
//   unit, each SIMD running one wave of each.
// * Key/value tiles of 64 keys are copied global -> LDS by buffer loads that
//   write LDS directly (no registers; rows past N arrive as zeros), double
//   buffered.  The loads of tile t+1 are spread over the S MFMAs of tile t
//   and waited for at the end of tile t, before the workgroup barrier.
// * LDS layout: both tiles row-major [key][d], 16-byte chunks XOR-swizzled
//   per row so that the operand reads below are free of bank conflicts (the
//   loads gather global chunks so that they land swizzled).
// * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: with K as the A operand (one
//   128-bit LDS read per fragment) and Q^T as the B operand, lane (g, j) of
//   the accumulator holds query j and 16 of the 32 keys of a block, so a
//   row's max and sum are in-register reductions plus one exchange between
//   the two half-waves (v_permlane32_swap).
// * O^T += V^T P^T on the same instruction: the probabilities leave the S
//   accumulator already in the B-operand layout of this product (the 16
//   accumulator rows of a lane are taken as the K index of the next MFMA),
//   so P never goes through LDS; the V^T operand comes straight out of the
//   row-major V tile through the LDS transpose read (ds_read_b64_tr_b16).
// * All K fragments of a tile are requested before its first MFMA and all
//   V^T fragments right after the last S MFMA, so each wave pays the LDS
//   latency once per operand and tile.
// * Causal: key tiles wholly in the future of the workgroup are never loaded
//   (loop bound), a wave whose 32 rows are all before a tile skips its math,
//   and only tiles that straddle the diagonal (or the ragged end of N) pay
//   for the element-wise mask (unit-12 causal-mask lesson: skip / diagonal /
//   past tiles).
// * Lazy base: a tile's probabilities are first computed against the row's
//   current exponent base, without a row maximum.  Only when some half-row
//   sum of the tile exceeds a bound (2^32 for bf16 probabilities, 2^15 for
//   fp16 ones), or is not finite -- always so on the first tile, whose base
//   is -inf -- does the wave take the slow path: row maximum, base moved to
//   it, accumulator and sum rescaled, probabilities recomputed.  Numerator
//   and denominator share the base, so O and the LSE are those of the exact
//   running maximum; the softmax of a tile costs no maximum on the fast path.
// * Grid: workgroups are dealt round-robin over the 8 XCDs; consecutive
//   workgroup ids are remapped so that each XCD walks a contiguous range of
//   heads (its 4 MB L2 then serves the K/V stream of one head to all its
//   query tiles).  Under the causal mask the longest query tiles of a head
//   are issued first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <type_traits>

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
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Element type of Q, K, V, O -- bf16 or fp16 -- with its gfx950 MFMA
// (32 x 32 x 16, fp32 accumulation) and vector types.
template <typename E>
struct Elem;
template <>
struct Elem<__bf16> {
    typedef bf16x8 x8;
    typedef bf16x4 x4;
    static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Elem<_Float16> {
    typedef f16x8 x8;
    typedef f16x4 x4;
    static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Row sums of the rounded probabilities, on the matrix core.  The output is
// normalised by the sum of exactly the (bf16 / fp16) probabilities that
// multiplied V, so numerator and denominator carry the same rounding; the LSE
// keeps the sum of the unrounded fp32 probabilities.  A P^T operand of
// O^T += V^T P^T (lane l: query l % 32, keys 8(l / 32) .. +7 of a 16-key step)
// is taken as the B operand of a 16 x 16 x 32 MFMA, which reads lane l as
// column l % 16, reduction index 8(l / 16) .. +7.  Columns thus hold query n
// in lane groups 0 and 2 and query n + 16 in groups 1 and 3; the 0/1 selector
// A (row m takes reduction group k / 8 when (m / 4) and (k / 8) have the same
// parity) makes output (m, n) the 16-key sum of query n (m / 4 even) or n + 16
// (m / 4 odd), and the output layout (lane l: column l % 16, rows
// 4(l / 16) .. +3) then gives every lane four copies of its own query's sum.
template <typename E>
__device__ __forceinline__ typename Elem<E>::x8 rowsum_selector(int lane) {
    typename Elem<E>::x8 a;
    const float one = ((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1)) ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (E)one;
    return a;
}

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBc = 64;                // keys per tile
// Largest half-row probability sum of a tile accepted against the current
// exponent base (every probability of the tile is then at most this): 2^32
// for bf16 probabilities (fp32's exponent range), 2^15 for fp16 ones (whose
// largest finite value is 65504).
template <typename E>
constexpr float kSumMax = 4294967296.f;
template <>
constexpr float kSumMax<_Float16> = 32768.f;

// Shared-memory tiles.  Both are [kBc keys][D] row-major, unpadded; the
// 16-byte chunks of a row are XOR-swizzled so that the MFMA operand reads hit
// distinct banks.  gfx950's LDS serves these reads 256 bytes at a time (16
// lanes of a 128-bit read, 32 lanes of a 64-bit read), so each group of
// chunks read together must land on 16 distinct 16-byte bank groups
// (measured with SQ_LDS_BANK_CONFLICT on candidate layouts):
//   K tile, read 16 rows x one chunk at a time:
//     d = 128: chunk c of row r stored at c ^ (r & 15);
//     d = 64 : two rows share a 256-byte line, chunk stored at c ^ ((r >> 1) & 7);
//   (both depend on r mod 32 only, so the reads of the second 32-row block
//   reuse the first block's offsets plus a constant);
//   V tile, read 4 rows x 4 chunks at a time by the transpose read:
//     d = 128: chunk stored at c ^ (4 * (r & 3));
//     d = 64 : chunk stored at c ^ (2 * (r & 3)).
// Tiles are filled by buffer loads that write LDS directly: lane l of a load
// instruction lands at LDS byte 16*l after the instruction's base, so the
// swizzle is applied on the global (gather) side.  Rows beyond N are outside
// the buffer's range and arrive as zeros.
//   d = 32 and d = 96 (also measured layouts of the same two read patterns,
//   checked conflict-free by enumeration):
//     K tile, d = 32 (four rows per 256-byte line): chunk c stored at
//       c ^ ((r >> 2) & 3);
//     K tile, d = 96 (192-byte rows, 12 chunks, where an XOR would leave the
//       row): chunk c stored at (c + 3 ((r >> 2) & 3)) mod 12;
//     V tile, d = 32 and 96: unswizzled (4 rows x 4 chunks already fall on 16
//       distinct bank groups, as 4r and 12r mod 16 step through multiples of 4).
template <int D>
__device__ __forceinline__ int k_swz(int r) {
    return D == 128 ? (r & 15) : D == 64 ? ((r >> 1) & 7) : D == 32 ? ((r >> 2) & 3) : 0;
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
    return D == 128 ? 4 * (r & 3) : D == 64 ? 2 * (r & 3) : 0;
}
// Stored chunk of logical chunk c in row r of a K tile, and the logical chunk
// stored at position p (the gather side of the tile copy).
template <int D>
__device__ __forceinline__ int k_stored(int r, int c) {
    if constexpr (D == 96) return (c + 3 * ((r >> 2) & 3)) % 12;
    else return c ^ k_swz<D>(r);
}
template <int D>
__device__ __forceinline__ int k_logical(int r, int p) {
    if constexpr (D == 96) return (p + 12 - 3 * ((r >> 2) & 3)) % 12;
    else return p ^ k_swz<D>(r);
}

#define LDS3 __attribute__((address_space(3)))

// Gather offset of a tile-copy lane with nothing to fetch: past the range of
// every descriptor the copies build (at most 2^31 bytes), so the lane's 16
// bytes arrive as zeros.
constexpr uint32_t kNoChunk = 0xFFFFFFF0u;

// Workgroup id -> (batch*head, query tile).  Consecutive ids go to
// consecutive XCDs.
//  * By default, when the grid divides evenly, XCD x receives the contiguous
//    range [x*W/8, (x+1)*W/8) of (head, tile) pairs, heavy tiles first
//    within a head under the causal mask: the XCD works through its heads
//    about one at a time and its L2 serves that head's K/V stream.
//  * Causal with fewer query tiles per head than `by_cost_below` (about
//    the workgroup slots of one XCD, so that many heads are in flight on an
//    XCD anyway): ids in order of decreasing cost, one cost rank after the
//    other over all heads -- largest first, so that the cheap tiles fill the
//    gaps left at the end of the grid (a makespan 22 % shorter at B16 H12
//    N1000 d64).  With a head count that is a multiple of 8, id mod 8 =
//    head mod 8: every tile of a head still runs on one XCD.  With long
//    rows this order measured 1 % faster at B2 H32 N8192 d128 but fetched
//    2.2x the HBM bytes (every head's K/V in flight at once), so long rows
//    keep the contiguous order.
__device__ __forceinline__ void map_block(int L, int W, int nqt, bool causal, int by_cost_below,
                                          int &bh, int &qt) {
    if (causal && nqt < by_cost_below) {
        const int heads = W / nqt;
        const int rank = L / heads;
        bh = L - rank * heads;
        qt = nqt - 1 - rank;
        return;
    }
    int gidx = L;
    if ((W & 7) == 0) {
        const int per = W >> 3;
        gidx = (L & 7) * per + (L >> 3);
    }
    bh = gidx / nqt;
    qt = gidx - bh * nqt;
    if (causal) qt = nqt - 1 - qt;
}

// Static schedules of the forward kernels.  Work item `it` of this
// workgroup: returns 0 when the workgroup has no more items, 1 with (bh, qt)
// set, 2 for a hole to skip.  Workgroup w runs on XCD w mod 8 (workgroups are
// dealt round-robin over the XCDs).  G = gridDim.x.
//  * mode 3: one tile per workgroup, the grid covering every tile, mapped by
//    map_block (the dispatcher balances the workgroups).
//  * mode 2 (persistent; the grid and the heads divide by 8): XCD x owns heads
//    x, x+8, ...; its L = G/8 workgroups take its (head, tile) items in rounds
//    of L, head-major with the longest causal tiles first, in snake order
//    (round r: workgroup lw takes item rL + lw, or rL + L-1-lw when r is odd).
//    Causal costs fall linearly along a head, so two consecutive rounds give
//    every workgroup the same work, and an XCD works on about one head at a
//    time, whose K/V its L2 then serves.
//  * mode 1 (persistent, causal): units are the tile pairs (nqt-1-i, i) of a
//    head, equal in cost, taken round-robin.
//  * mode 0 (persistent): single tiles round-robin, longest causal tiles
//    first over all heads.
// No atomics and no dispatcher involvement after the launch in modes 0-2.
__device__ __forceinline__ int sched_item(int mode, int it, int n_bh, int nqt, bool causal,
                                          int by_cost_below, int &bh, int &qt) {
    const int G = gridDim.x;
    if (mode == 3) {
        if (it > 0) return 0;
        map_block(blockIdx.x, G, nqt, causal, by_cost_below, bh, qt);
        return 1;
    }
    const int L = G >> 3;
    const int x = blockIdx.x & 7, lw = blockIdx.x >> 3;
    if (mode == 2) {
        const int n_local = (n_bh >> 3) * nqt;
        if (it * L >= n_local) return 0;
        const int pos = it * L + ((it & 1) ? (L - 1 - lw) : lw);
        if (pos >= n_local) return 2;
        const int lh = pos / nqt, pq = pos - lh * nqt;
        bh = lh * 8 + x;
        qt = causal ? nqt - 1 - pq : pq;
        return 1;
    }
    const int slot = ((G & 7) == 0) ? x * L + lw : (int)blockIdx.x;
    if (mode == 1) {
        const int npairs = (nqt + 1) / 2;
        const int unit = slot + (it >> 1) * G;
        if (unit >= n_bh * npairs) return 0;
        bh = unit / npairs;
        const int pi = unit - bh * npairs;
        if (it & 1) {
            if (nqt - 1 - pi == pi) return 2;  // the middle tile of an odd count
            qt = pi;
        } else {
            qt = nqt - 1 - pi;
        }
        return 1;
    }
    const int unit = slot + it * G;
    if (unit >= n_bh * nqt) return 0;
    if (causal) {
        const int rank = unit / n_bh;
        bh = unit - rank * n_bh;
        qt = nqt - 1 - rank;
    } else {
        bh = unit / nqt;
        qt = unit - bh * nqt;
    }
    return 1;
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Buffer descriptor over `bytes` bytes starting at `base` (raw, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Enqueue load number i (0 <= i < 2 kLoads) of the next key tile (keys c0 ..
// c0 + kBc - 1): even i load K into dk, odd i load V into dv, load u = i/2
// of this wave's share, one 16-byte direct-to-LDS load per lane.  Rows at or
// beyond N read as zeros.  The loads of a tile are issued one at a time
// between the MFMAs of the tile being computed: issued as one burst by every
// wave, they fill the texture-address queue and the in-order wave stalls
// behind them before it can start its MFMAs.  (Kept out of the kernel's
// lambdas: a buffer descriptor local in a lambda makes the host pass drop the
// kernel's launch stub.)
// Strided views (STRIDED): rows of K and V are kn and vn elements apart; the
// descriptor then ends after the last valid row's d elements.
template <int DH, int kLoads, bool STRIDED, typename E>
__device__ __forceinline__ void issue_tile_load(int i, const E *Kh, const E *Vh, int N, int c0,
                                                LDS3 char *dk, LDS3 char *dv,
                                                const uint32_t *k_src, const uint32_t *v_src,
                                                int wave, int kn, int vn) {
    const int u = i >> 1;
    const int pos = (u * kWaves + wave) * 64 * 16;  // byte offset of this wave's 1 KiB
    if constexpr (!STRIDED) {
        const uint32_t bytes = (uint32_t)min(kBc, N - c0) * (uint32_t)(DH * 2);
        if ((i & 1) == 0) {
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)c0 * DH, bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS3 void *)(dk + pos), 16, k_src[u], 0, 0, 0);
        } else {
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)c0 * DH, bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS3 void *)(dv + pos), 16, v_src[u], 0, 0, 0);
        }
    } else {
        const uint32_t rows = (uint32_t)min(kBc, N - c0);
        if ((i & 1) == 0) {
            const uint32_t bytes = (rows - 1) * (uint32_t)kn * 2u + (uint32_t)(DH * 2);
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)c0 * kn, bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LDS3 void *)(dk + pos), 16, k_src[u], 0, 0, 0);
        } else {
            const uint32_t bytes = (rows - 1) * (uint32_t)vn * 2u + (uint32_t)(DH * 2);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)c0 * vn, bytes);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LDS3 void *)(dv + pos), 16, v_src[u], 0, 0, 0);
        }
    }
}

// Element strides of strided views (d is contiguous); LSE stays [B, H, N].
struct FwdStrides {
    long long qb, qh, kb, kh, vb, vh, ob, oh;
    int qn, kn, vn, on, H;
};

// OCC: waves per SIMD the kernel is compiled for (2, or 3 at d = 64: 168
// registers instead of 176, three workgroups per compute unit).
template <typename E, int DH, bool CAUSAL, bool STRIDED, int OCC = 2>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
fwd_kernel(const E *__restrict__ Q, const E *__restrict__ K, const E *__restrict__ V,
           E *__restrict__ O, float *__restrict__ LSE, int N, int nqt, int n_bh, int mode,
           float scale, float scale_log2, FwdStrides st) {
    typedef typename Elem<E>::x8 X8;
    typedef typename Elem<E>::x4 X4;
    static_assert(DH % 16 == 0 && DH >= 16 && DH <= 128, "head dim");
    // A head dim that is an odd multiple of 16 runs in the layout of the next
    // multiple of 32 (D): S takes DH / 16 k-steps, the LDS tiles and the O^T
    // blocks have D / 32 d-blocks, and the tile copies write zeros into the
    // chunks at and past DH (their O^T rows are computed but never stored).
    constexpr int D = (DH + 31) / 32 * 32;
    constexpr int KS = DH / 16;                                 // k-steps of S^T = K Q^T
    constexpr int kChunksPerRow = D / 8;                        // 16-byte chunks
    constexpr int kLoads = kBc * kChunksPerRow / kThreads;     // per thread per tile
    // Two buffers per operand as four distinct objects: the tile loop is
    // unrolled by two so that every access names its buffer at compile time,
    // which lets the compiler see that the loads filling one buffer do not
    // touch the one being read (no wait on the in-flight loads).
    __shared__ __attribute__((aligned(16))) __bf16 lds_k0[kBc * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_k1[kBc * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v0[kBc * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v1[kBc * D];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 5;  // half-wave
    const int j = lane & 31;  // query column of this lane (S^T / O^T layouts)

    int qn, kn, vn, on;  // row strides (elements)
    if constexpr (STRIDED) {
        qn = st.qn;
        kn = st.kn;
        vn = st.vn;
        on = st.on;
    } else {
        qn = kn = vn = on = DH;
    }
    // ---- staging offsets (lane constants) ---------------------------------
    // Load u of wave w fills LDS chunk positions [(u*kWaves + w)*64, +64); lane l
    // fills position q = that base + l, i.e. row q / kChunksPerRow, stored
    // chunk q % kChunksPerRow, and must fetch the logical chunk that the
    // swizzle puts there.
    // A position whose logical chunk lies at or past DH gets an offset past
    // any descriptor's range, so the copy writes zeros there.
    uint32_t k_src[kLoads], v_src[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        const int q = (u * kWaves + wave) * 64 + lane;
        const int r = q / kChunksPerRow;
        const int p = q % kChunksPerRow;
        const int ck = k_logical<D>(r, p), cv = p ^ v_swz<D>(r);
        k_src[u] = (DH == D || ck < DH / 8) ? (uint32_t)(r * kn * 2 + (ck << 4)) : kNoChunk;
        v_src[u] = (DH == D || cv < DH / 8) ? (uint32_t)(r * vn * 2 + (cv << 4)) : kNoChunk;
    }
    // The 2 kLoads tile loads are spread evenly over the KS k-steps of S:
    // k-step ks issues loads [ks L / KS, (ks + 1) L / KS), L = 2 kLoads.
    constexpr int kTileLoads = 2 * kLoads;

    // MFMA operand read offsets (bytes within a tile).
    // K (A operand of S^T = K Q^T): lane (g, j) reads row 32kb + j, logical
    // chunk 2ks + g.
    uint32_t k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        k_rd[ks] = (uint32_t)(j * D * 2 + (k_stored<D>(j, 2 * ks + g) << 4));
    // V^T (A operand of O^T += V^T P^T) through the 16-lane transpose read:
    // in group G = lane/16 (m0 = 16*(G&1), g = G>>1), lane i of the group reads
    // row 16T + 8h + 4g + i/4, columns 32db + m0 + 4(i%4) .. +3.  The row's
    // low two bits are i/4, so the swizzle term is a lane constant and the
    // offset depends on db only through the stored chunk.
    const int gi = lane & 15;
    const int m0 = 16 * ((lane >> 4) & 1);
    uint32_t v_rd[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int row = 4 * g + (gi >> 2);
        const int col = 32 * db + m0 + 4 * (gi & 3);
        const int c = col >> 3;
        v_rd[db] = (uint32_t)(row * D * 2 + ((c ^ v_swz<D>(row)) << 4) + ((col & 4) << 1));
    }

    const X8 sel = rowsum_selector<E>(lane);
    LDS3 char *const k0 = (LDS3 char *)lds_k0;
    LDS3 char *const k1 = (LDS3 char *)lds_k1;
    LDS3 char *const v0 = (LDS3 char *)lds_v0;
    LDS3 char *const v1 = (LDS3 char *)lds_v1;

    // Work items: see sched_item (mode 3: one tile, from map_block).
    for (int it = 0;; ++it) {
        int bh, qt;
        const int got = sched_item(mode, it, n_bh, nqt, CAUSAL, 64, bh, qt);
        if (got == 0) break;
        if (got == 2) continue;
        {
            // The previous tile's LDS buffers are free and its copies landed.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const int r0 = qt * kBr;
            size_t qoff, koff, voff, ooff;
            if constexpr (STRIDED) {
                const int b = bh / st.H, h = bh - b * st.H;
                qoff = (size_t)(b * st.qb + h * st.qh);
                koff = (size_t)(b * st.kb + h * st.kh);
                voff = (size_t)(b * st.vb + h * st.vh);
                ooff = (size_t)(b * st.ob + h * st.oh);
            } else {
                qoff = koff = voff = ooff = (size_t)bh * (size_t)N * DH;
            }
            const E *Qh = Q + qoff;
            const E *Kh = K + koff;
            const E *Vh = V + voff;
            const int wrow0 = r0 + wave * kRowsPerWave;
            const int qrow = wrow0 + j;

            // Q^T as the B operand: lane (g, j) holds query qrow, columns 16ks+8g..+7.
            X8 qop[KS];
        #pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (qrow < N) x = load16(Qh + (size_t)qrow * qn + 16 * ks + 8 * g);
                qop[ks] = __builtin_bit_cast(X8, x);
            }

            const int kv_end = CAUSAL ? min(N, r0 + kBr) : N;
            const int n_tiles = (kv_end + kBc - 1) / kBc;

            f32x16 acc[D / 32];
        #pragma unroll
            for (int db = 0; db < D / 32; ++db)
        #pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
            float m_run = -INFINITY;  // exponent base of row qrow (raw score units)
            float mc_run = -INFINITY; // the base in scaled log2 units (m_run * scale_log2)
            float l_run = 0.f;        // this half-wave's share of the running sum
            float lr_run = 0.f;       // running sum of the rounded probabilities (whole row)


            // One key tile: prefetch the next tile into the other buffers, then
            // S^T, softmax and O^T on this one.
            auto step = [&](int t, const LDS3 char *kt, const LDS3 char *vt, LDS3 char *nk,
                            LDS3 char *nv) {
                const int c0 = t * kBc;
                const bool prefetch = t + 1 < n_tiles;
                auto load = [&](int i) __attribute__((always_inline)) {
                    issue_tile_load<DH, kLoads, STRIDED>(i, Kh, Vh, N, c0 + kBc, nk, nv, k_src, v_src,
                                                         wave, kn, vn);
                };

                // Checking build: the next tile is copied and visible before this
                // tile's compute starts (its buffers were released at the barrier
                // that ended the previous tile).
                if constexpr (kSafeSync) {
                    if (prefetch) {
        #pragma unroll
                        for (int i = 0; i < 2 * kLoads; ++i) load(i);
                    }
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
                }
                // A wave whose rows all precede this tile has nothing to add.
                const bool active = !CAUSAL || c0 <= wrow0 + kRowsPerWave - 1;
                if (!active && prefetch && !kSafeSync) {
        #pragma unroll
                    for (int i = 0; i < 2 * kLoads; ++i) load(i);
                }
                if (active) {

                    // S^T[key][query] = K Q^T for the kBc keys of this tile.
                    f32x16 s[kBc / 32];
        #pragma unroll
                    for (int kb = 0; kb < kBc / 32; ++kb)
        #pragma unroll
                        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
                    // All K fragments of the tile are requested before the first MFMA,
                    // so the LDS latency is paid once per tile, not once per k-step.
                    X8 kf[KS][kBc / 32];
        #pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
        #pragma unroll
                        for (int kb = 0; kb < kBc / 32; ++kb)
                            kf[ks][kb] = *reinterpret_cast<const LDS3 X8 *>(
                                kt + k_rd[ks] + kb * 32 * D * 2);
                    __builtin_amdgcn_sched_barrier(0);
                    // The S MFMAs run at raised wave priority: the other wave on this
                    // SIMD (from another workgroup) then tends to run its softmax while
                    // this one keeps the matrix core busy, instead of both waves
                    // alternating instruction by instruction through the same phase.
                    __builtin_amdgcn_s_setprio(1);
                    // The next tile's loads go out one per k-step, between the MFMAs.
        #pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
        #pragma unroll
                        for (int kb = 0; kb < kBc / 32; ++kb)
                            s[kb] = Elem<E>::mfma(kf[ks][kb], qop[ks], s[kb]);
                        if (prefetch && !kSafeSync) {
        #pragma unroll
                            for (int i = ks * kTileLoads / KS; i < (ks + 1) * kTileLoads / KS; ++i) load(i);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }

                    __builtin_amdgcn_s_setprio(0);

                    // All V^T fragments of the tile are requested now; the softmax below
                    // covers their latency.  Fragment (T, db) is two transpose reads
                    // (keys 16T+4g+k and 16T+8+4g+k, columns of d-block db).
                    X8 vf[kBc / 16][D / 32];
        #pragma unroll
                    for (int T = 0; T < kBc / 16; ++T)
        #pragma unroll
                        for (int db = 0; db < D / 32; ++db) {
                            const LDS3 char *base = vt + v_rd[db] + T * 16 * D * 2;
                            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 v4i16 *)(base));
                            const v4i16 hi =
                                __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 v4i16 *)(base + 8 * D * 2));
                            vf[T][db] = __builtin_bit_cast(
                                X8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        }

                    // Element r of s[kb] is key c0 + 32kb + 8(r/4) + 4g + r%4.
                    const bool need_mask = (CAUSAL && c0 + kBc - 1 > wrow0) || (c0 + kBc > N);
                    if (need_mask) {
                        // visible iff 32kb + 8(r/4) + r%4 <= lim, lim = min(qrow, N-1) - c0 - 4g
                        const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - c0 - 4 * g;
        #pragma unroll
                        for (int kb = 0; kb < kBc / 32; ++kb)
        #pragma unroll
                            for (int r = 0; r < 16; ++r)
                                if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
                    }

                    // Fast path: probabilities against the current exponent base, with
                    // no row maximum.  The tile is accepted when every half-row sum is
                    // at most kSumMax (so every probability is); the test also rejects
                    // inf / NaN sums, in particular on the first tile, whose base is
                    // still -inf.  Numerator and denominator share the base, so
                    // O = acc / l and LSE = base*scale + ln(l) do not depend on where
                    // the base sits.
                    X8 pop[kBc / 16];
                    float rs = 0.f;
                    auto exps = [&](float mcx) __attribute__((always_inline)) {
                        rs = 0.f;
        #pragma unroll
                        for (int kb = 0; kb < kBc / 32; ++kb) {
                            f32x8 lo, hi;
        #pragma unroll
                            for (int r = 0; r < 8; ++r) {
                                lo[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], scale_log2, -mcx));
                                hi[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 8], scale_log2, -mcx));
                                rs += lo[r];
                                rs += hi[r];
                            }
                            pop[2 * kb] = __builtin_convertvector(lo, X8);
                            pop[2 * kb + 1] = __builtin_convertvector(hi, X8);
                        }
                    };
                    // The first tile of a work item (t = 0) always takes the slow
                    // path (the base is still -inf), so it skips the attempt.
                    bool slow = t == 0;
                    if (!slow) {
                        exps(mc_run);
                        slow = __ballot(!(rs <= kSumMax<E>)) != 0;
                    }
                    if (slow) {
                        // Slow path: the base moves to the row maximum (tile and
                        // running), the accumulator and sum are rescaled, and the
                        // tile's probabilities are recomputed against the new base.
                        float mt = s[0][0];
        #pragma unroll
                        for (int kb = 0; kb < kBc / 32; ++kb)
        #pragma unroll
                            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
                        {
                            const auto sw = __builtin_amdgcn_permlane32_swap(
                                __float_as_uint(mt), __float_as_uint(mt), false, false);
                            mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                        }
                        const float m_new = fmaxf(m_run, mt);
                        // A row that has seen no visible key keeps base 0 (its terms are 0).
                        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                        const float alpha = (m_run == -INFINITY) ? 0.f
                                                                 : __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
                        mc_run = m_use * scale_log2;
                        m_run = m_use;
                        l_run *= alpha;
        #pragma unroll
                        for (int db = 0; db < D / 32; ++db)
        #pragma unroll
                            for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
                        lr_run *= alpha;
                        exps(mc_run);
                    }
                    l_run += rs;

                    // O^T[d][query] += V^T P^T; k-step T covers keys 16T..16T+15.
        #pragma unroll
                    for (int T = 0; T < kBc / 16; ++T)
        #pragma unroll
                        for (int db = 0; db < D / 32; ++db)
                            acc[db] = Elem<E>::mfma(vf[T][db], pop[T], acc[db]);
                    f32x4 lt = {0.f, 0.f, 0.f, 0.f};
        #pragma unroll
                    for (int T = 0; T < kBc / 16; ++T) lt = Elem<E>::mfma16(sel, pop[T], lt);
                    lr_run += lt[0];
                }

                // The next tile's loads must have landed before anyone reads them, and
                // every wave must be done with this tile before it is overwritten.
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            };

        #pragma unroll
            for (int i = 0; i < 2 * kLoads; ++i)
                issue_tile_load<DH, kLoads, STRIDED>(i, Kh, Vh, N, 0, k0, v0, k_src, v_src, wave, kn, vn);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            for (int t = 0; t < n_tiles; t += 2) {
                step(t, k0, v0, k1, v1);
                if (t + 1 < n_tiles) step(t + 1, k1, v1, k0, v0);
            }

            // Epilogue: O = acc / (sum of the rounded probabilities), rounded to the
            // element type; LSE = m*scale + ln(l) with the fp32 sum l.
            float l_tot;
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                                 __float_as_uint(l_run), false, false);
                l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            const float inv = 1.f / lr_run;
            if (qrow < N) {
                E *orow = O + ooff + (size_t)qrow * on;
        #pragma unroll
                for (int db = 0; db < D / 32; ++db)
        #pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int col = 32 * db + 8 * a + 4 * g;
                        if (DH % 32 != 0 && col >= DH) continue;
                        f32x4 x;
        #pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * a + e] * inv;
                        *reinterpret_cast<X4 *>(orow + col) = __builtin_convertvector(x, X4);
                    }
                if (g == 0) LSE[(size_t)bh * N + qrow] = m_run * scale + logf(l_tot);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Software-pipelined kernel (head dims 64 and 128), W waves of 32 query rows
// per workgroup.
//
// Same operand layouts, LDS swizzles and lazy exponent base as fwd_kernel
// above; what changes is the order of work inside a wave.  The key axis is
// walked in 32-key half tiles h, and step h of a wave issues, as one
// interleaved instruction stream,
//   * the O^T += V^T P^T MFMAs of half tile h-1,
//   * the S^T = K Q^T MFMAs of half tile h+1, and
//   * the softmax of half tile h (VALU), whose scores came out of step h-1,
// none of which depends on another within the step.  The matrix core then
// runs while the same wave computes its exponentials, so the overlap no
// longer depends on the two waves of a SIMD being in opposite phases; that
// in turn allows workgroups of 8 waves (256 query rows), which halves the
// L2 -> LDS tile stream per FLOP.  The LDS reads of a step's first two MFMA
// pairs are issued at the end of the step before, so that no step starts
// by waiting for LDS.
//
// Every step runs the same straight-line code (a wave past its last
// visible key multiplies zero probabilities until the workgroup's tiles
// run out, or leaves the loop once it has added its last probabilities;
// a half tile with masked keys takes a short masking branch first), so the
// accumulators keep their registers from step to step.
//
// Buffers: three per operand; K tile i and V tile i live in buffer i mod 3.
// A 64-key tile spans two steps: tile step t (steps 2t+1, 2t+2) reads V(t)
// and K(t+1) and copies K(t+3) and V(t+2) into the buffers of K(t) and
// V(t-1), which were last read in tile step t-1.  One barrier at the top of
// each tile step orders those overwrites; each wave's copies have landed
// (vmcnt) before it meets the barrier, so a tile copied in tile step t is
// visible to all waves from tile step t+1 on, one tile step before it is
// read -- which lets the end of tile step t read ahead into tile step t+1.
constexpr int kPipeBufs = 3;

// One 16-byte direct-to-LDS load per lane (load u of this wave's share) of
// a tile with `rows` valid rows at `base` (row stride rs elements), for a
// workgroup of W waves.  Load u covers tile rows from u R on, R = 64 W / (D /
// 8); at D = 64 and 128 the swizzle of a row depends on its index modulo 32
// and 16 only, so the lane's gather offset `src` (that of load 0) serves
// every load, with the descriptor's base moved to row u R and its size cut
// to the rows that remain (the hardware range check turns every row at or
// past `rows` into zeros; none remaining gives an empty range and a load of
// zeros only).
template <int D, int W, bool STRIDED, typename E>
__device__ __forceinline__ void tile_load(const E *base, int rows, int rs, LDS3 char *dst,
                                          uint32_t src, int u, int wave) {
    static_assert(D == 64 || D == 128, "row swizzle periodic in the load's row step");
    constexpr int kRowsPerLoad = 64 * W / (D / 8);
    const int pos = (u * W + wave) * 64 * 16;
    const int left = rows - u * kRowsPerLoad;
    uint32_t bytes = 0;
    if (left > 0)
        bytes = STRIDED ? (uint32_t)(left - 1) * (uint32_t)rs * 2u + (uint32_t)(D * 2)
                        : (uint32_t)left * (uint32_t)(D * 2);
    // (The size is wave-uniform; said explicitly, as the compiler may
    // otherwise clamp it in a vector register and wrap the load in a loop
    // over distinct descriptors.)
    bytes = __builtin_amdgcn_readfirstlane(bytes);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (size_t)u * kRowsPerLoad * rs, bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS3 void *)(dst + pos), 16, src, 0, 0, 0);
}

template <typename E, int D, bool CAUSAL, bool STRIDED, int W>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_pipe_kernel(const E *__restrict__ Q, const E *__restrict__ K, const E *__restrict__ V,
                E *__restrict__ O, float *__restrict__ LSE, int N, int nqt, int n_bh, int mode,
                float scale, float scale_log2, FwdStrides st) {
    typedef typename Elem<E>::x8 X8;
    typedef typename Elem<E>::x4 X4;
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(W == 4 || W == 8, "waves");
    // Two workgroups share a compute unit at W = 4: their six tiles of each
    // operand must fit its 160 KiB of LDS.
    static_assert(W == 8 || 2 * 2 * kPipeBufs * kBc * D * 2 <= 160 * 1024, "LDS");
    constexpr int kRows = W * kRowsPerWave;   // query rows per workgroup
    constexpr int kChunksPerRow = D / 8;
    constexpr int kLoads = kBc * kChunksPerRow / (64 * W);  // per operand and lane
    constexpr int KS = D / 16;  // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;  // 32-wide d blocks of O^T
    static_assert(2 * DB == KS, "one P V^T MFMA per K Q^T MFMA");
    __shared__ __attribute__((aligned(16))) __bf16 lds_k0[kBc * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_k1[kBc * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_k2[kBc * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v0[kBc * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v1[kBc * D];
    __shared__ __attribute__((aligned(16))) __bf16 lds_v2[kBc * D];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 5;
    const int j = lane & 31;

    int qn, kn, vn, on;  // row strides (elements)
    if constexpr (STRIDED) {
        qn = st.qn;
        kn = st.kn;
        vn = st.vn;
        on = st.on;
    } else {
        qn = kn = vn = on = D;
    }
    // Gather offsets of the lane's first tile load (see tile_load).
    uint32_t k_src, v_src;
    {
        const int q = wave * 64 + lane;
        const int r = q / kChunksPerRow;
        const int p = q % kChunksPerRow;
        k_src = (uint32_t)(r * kn * 2 + (k_logical<D>(r, p) << 4));
        v_src = (uint32_t)(r * vn * 2 + ((p ^ v_swz<D>(r)) << 4));
    }
    uint32_t k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        k_rd[ks] = (uint32_t)(j * D * 2 + (k_stored<D>(j, 2 * ks + g) << 4));
    const int gi = lane & 15;
    const int m0 = 16 * ((lane >> 4) & 1);
    uint32_t v_rd[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int row = 4 * g + (gi >> 2);
        const int col = 32 * db + m0 + 4 * (gi & 3);
        const int c = col >> 3;
        v_rd[db] = (uint32_t)(row * D * 2 + ((c ^ v_swz<D>(row)) << 4) + ((col & 4) << 1));
    }

    const X8 sel = rowsum_selector<E>(lane);
    LDS3 char *const kb[kPipeBufs] = {(LDS3 char *)lds_k0, (LDS3 char *)lds_k1,
                                      (LDS3 char *)lds_k2};
    LDS3 char *const vb[kPipeBufs] = {(LDS3 char *)lds_v0, (LDS3 char *)lds_v1,
                                      (LDS3 char *)lds_v2};

    // Work items: see sched_item.
    for (int it = 0;; ++it) {
        int bh, qt;
        const int got = sched_item(mode, it, n_bh, nqt, CAUSAL, 32 * (8 / W), bh, qt);
        if (got == 0) break;
        if (got == 2) continue;
        {
            // Every wave is done with the previous tile's LDS buffers (and
            // its copies have landed) before this tile's prologue refills them.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const int r0 = qt * kRows;
            size_t qoff, koff, voff, ooff;
            if constexpr (STRIDED) {
                const int b = bh / st.H, h = bh - b * st.H;
                qoff = (size_t)(b * st.qb + h * st.qh);
                koff = (size_t)(b * st.kb + h * st.kh);
                voff = (size_t)(b * st.vb + h * st.vh);
                ooff = (size_t)(b * st.ob + h * st.oh);
            } else {
                qoff = koff = voff = ooff = (size_t)bh * (size_t)N * D;
            }
            const E *Qh = Q + qoff;
            const E *Kh = K + koff;
            const E *Vh = V + voff;
            const int wrow0 = r0 + wave * kRowsPerWave;
            const int qrow = wrow0 + j;

            X8 qop[KS];
        #pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (qrow < N) x = load16(Qh + (size_t)qrow * qn + 16 * ks + 8 * g);
                qop[ks] = __builtin_bit_cast(X8, x);
            }

            const int kv_end = CAUSAL ? min(N, r0 + kRows) : N;
            const int n_tiles = (kv_end + kBc - 1) / kBc;
            // Row qrow sees keys 0 .. vis (the element mask below); the wave's rows
            // see keys up to vis_max at most.
            const int vis = CAUSAL ? min(qrow, N - 1) : N - 1;
            const int vis_max = CAUSAL ? wrow0 + kRowsPerWave - 1 : N - 1;

            f32x16 acc[DB];
        #pragma unroll
            for (int db = 0; db < DB; ++db)
        #pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
            float m_run = -INFINITY;   // exponent base of row qrow (raw score units)
            float mc_run = -INFINITY;  // the base times scale * log2(e)
            float l_run = 0.f;         // this half-wave's share of the running sum
            float lr_run = 0.f;        // running sum of the rounded probabilities (whole row)


            // LDS reads of MFMA pair i of a step: the V^T fragment (i / DB, i % DB)
            // of half `hv` of tile buffer vt (two transpose reads) and the K
            // fragment of k-step i of half `hk` of tile buffer kt.
            auto read_pair = [&](int i, const LDS3 char *kt, int hk, const LDS3 char *vt, int hv, X8 &vfr,
                                 X8 &kfr) __attribute__((always_inline)) {
                const LDS3 char *base = vt + v_rd[i % DB] + (2 * hv + i / DB) * 16 * D * 2;
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 v4i16 *)(base));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 v4i16 *)(base + 8 * D * 2));
                vfr = __builtin_bit_cast(X8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                kfr = *reinterpret_cast<const LDS3 X8 *>(kt + k_rd[i] + hk * 32 * D * 2);
            };

            // Element r of a half tile's S^T block is key 32h + 8(r/4) + 4g + r%4 of
            // query qrow; its P^T operands p[0], p[1] cover keys 32h .. +15 and
            // 32h+16 .. +31 (k-steps of O^T += V^T P^T).
            //
            // Probabilities of one half tile against exponent base mcx (scaled log2
            // units) as P^T operands, and their (half-wave) sum.
            auto exps = [&](const f32x16 &s, float mcx, X8 (&p)[2]) __attribute__((always_inline)) {
                f32x8 lo, hi;
                float ra = 0.f, rb = 0.f;
        #pragma unroll
                for (int r = 0; r < 8; ++r) {
                    lo[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -mcx));
                    hi[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 8], scale_log2, -mcx));
                    ra += lo[r];
                    rb += hi[r];
                }
                p[0] = __builtin_convertvector(lo, X8);
                p[1] = __builtin_convertvector(hi, X8);
                return ra + rb;
            };
            // Slow path of the lazy base: the base moves to the row maximum, the
            // accumulator and the sum are rescaled, the probabilities recomputed.
            auto rebase = [&](const f32x16 &s, X8 (&p)[2]) __attribute__((always_inline)) {
                float mt = s[0];
        #pragma unroll
                for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
                {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                                     false, false);
                    mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                }
                const float m_new = fmaxf(m_run, mt);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha =
                    (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
                mc_run = m_use * scale_log2;
                m_run = m_use;
                l_run *= alpha;
        #pragma unroll
                for (int db = 0; db < DB; ++db)
        #pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
                lr_run *= alpha;
                return exps(s, mc_run, p);
            };

            // Step h.  (kt, hk): LDS tile buffer and half holding the K rows of half
            // tile h+1; (vt, hv): those holding the V rows of half tile h-1;
            // (ktn, hkn), (vtn, hvn): the same for step h+1, whose first two MFMA
            // pairs' operands this step reads at its end.  vf0/kf0: this step's
            // first two pairs' operands (in), the next step's (out).  sc: scores of
            // half tile h (in), sn: scores of half tile h+1 (out); pp: P^T of half
            // tile h-1 (in), pc: P^T of half tile h (out).  With LOADS, the step
            // also issues the copies of K(t+3) into kload and V(t+2) into vload
            // (t = the tile of half tile h).  Every buffer a step reads has been
            // filled (possibly with zeros past kv_end), so steps outside the wave's
            // visible range compute finite, discarded scores and add zero
            // probabilities.
            auto step = [&](int h, auto loads_tag, const LDS3 char *kt, int hk, const LDS3 char *vt, int hv,
                            const LDS3 char *ktn, int hkn, const LDS3 char *vtn, int hvn,
                            LDS3 char *kload, LDS3 char *vload, X8 (&vf0)[2], X8 (&kf0)[2], f32x16 &sc,
                            f32x16 &sn, X8 (&pp)[2], X8 (&pc)[2]) __attribute__((always_inline)) {
                constexpr bool LOADS = decltype(loads_tag)::value;
                // Element mask of half tile h: visible iff 8(r/4) + r%4 <= lim.
                const int lim = vis - 32 * h - 4 * g;
                if (32 * h + 31 > (CAUSAL ? wrow0 : N - 1)) {
        #pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) > lim) sc[r] = -INFINITY;
                }
                // MFMA pair i: P V^T with V^T fragment (i / DB, i % DB), then K Q^T
                // k-step i.  LDS reads in the order of use: pairs 2 .. KS-1 of this
                // step, then pairs 0, 1 of the next.
                X8 vf[KS], kf[KS];
                vf[0] = vf0[0];
                kf[0] = kf0[0];
                vf[1] = vf0[1];
                kf[1] = kf0[1];
        #pragma unroll
                for (int i = 2; i < KS; ++i) read_pair(i, kt, hk, vt, hv, vf[i], kf[i]);
                read_pair(0, ktn, hkn, vtn, hvn, vf0[0], kf0[0]);
                read_pair(1, ktn, hkn, vtn, hvn, vf0[1], kf0[1]);
        #pragma unroll
                for (int r = 0; r < 16; ++r) sn[r] = 0.f;
                // Row sums of P^T of half tile h-1 (the operands of this step's
                // P V^T), added to the running sum at the end of the step.
                f32x4 lt = {0.f, 0.f, 0.f, 0.f};
                lt = Elem<E>::mfma16(sel, pp[0], lt);
                lt = Elem<E>::mfma16(sel, pp[1], lt);
        #pragma unroll
                for (int i = 0; i < KS; ++i) {
                    acc[i % DB] = Elem<E>::mfma(vf[i], pp[i / DB], acc[i % DB]);
                    sn = Elem<E>::mfma(kf[i], qop[i], sn);
                }
                float rs = exps(sc, mc_run, pc);
                if constexpr (LOADS) {
                    const int t = h >> 1;
                    const E *kbase = Kh + (size_t)(t + 3) * kBc * kn;
                    const E *vbase = Vh + (size_t)(t + 2) * kBc * vn;
                    const int krows = min(kBc, kv_end - (t + 3) * kBc);
                    const int vrows = min(kBc, kv_end - (t + 2) * kBc);
        #pragma unroll
                    for (int u = 0; u < kLoads; ++u) {
                        tile_load<D, W, STRIDED>(kbase, krows, kn, kload, k_src, u, wave);
                        tile_load<D, W, STRIDED>(vbase, vrows, vn, vload, v_src, u, wave);
                    }
                }
                // Per pair: the three LDS reads of the pair two ahead (of the next
                // step for the last two pairs), then each MFMA followed by its share
                // of the softmax; the tile copies spread evenly.
                constexpr int kValu = (56 + 2 * KS - 1) / (2 * KS);  // softmax VALU per MFMA
                constexpr int kCopyEvery = KS / (2 * kLoads);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // the two row-sum MFMAs
        #pragma unroll
                for (int i = 0; i < KS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
                    if (LOADS && i % kCopyEvery == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                lr_run += lt[0];  // before a rebase, which rescales it with acc
                if (__ballot(!(rs <= kSumMax<E>))) rs = rebase(sc, pc);
                l_run += rs;
            };

            f32x16 sA, sB;
            X8 pA[2], pB[2] = {X8{}, X8{}};
            X8 vf0[2], kf0[2];
            const std::integral_constant<bool, true> with_loads;
            const std::integral_constant<bool, false> no_loads;

            // Prologue: K(0), K(1), K(2), V(0), V(1) into LDS (tile step t copies
            // K(t+3) and V(t+2)); scores of half tile 0; step 0 (whose P V^T adds
            // zeros).
        #pragma unroll
            for (int u = 0; u < kLoads; ++u) {
        #pragma unroll
                for (int i = 0; i < 3; ++i)
                    tile_load<D, W, STRIDED>(Kh + (size_t)i * kBc * kn, min(kBc, kv_end - i * kBc), kn, kb[i],
                                             k_src, u, wave);
        #pragma unroll
                for (int i = 0; i < 2; ++i)
                    tile_load<D, W, STRIDED>(Vh + (size_t)i * kBc * vn, min(kBc, kv_end - i * kBc), vn, vb[i],
                                             v_src, u, wave);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            {
                X8 kf[KS];
        #pragma unroll
                for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const LDS3 X8 *>(kb[0] + k_rd[ks]);
        #pragma unroll
                for (int r = 0; r < 16; ++r) sA[r] = 0.f;
        #pragma unroll
                for (int ks = 0; ks < KS; ++ks) sA = Elem<E>::mfma(kf[ks], qop[ks], sA);
            }
            read_pair(0, kb[0], 1, vb[0], 0, vf0[0], kf0[0]);
            read_pair(1, kb[0], 1, vb[0], 0, vf0[1], kf0[1]);
            // Step 0 reads K half tile 1 (tile 0, half 1); step 1 reads K tile 1
            // half 0 and V tile 0 half 0.
            step(0, no_loads, kb[0], 1, vb[0], 0, kb[1], 0, vb[0], 0, kb[0], vb[0], vf0, kf0, sA, sB, pB, pA);

            // Tile step t (buffers b = t mod 3): step 2t+1 reads K(t+1) half 0 and
            // V(t) half 0, step 2t+2 their halves 1, and step 2t+3 (read ahead) K(t+2)
            // half 0 and V(t+1) half 0.  A wave whose last visible half tile hlast
            // has had its P V^T (step hlast+1) leaves the loop; for the rest of the
            // workgroup's tiles it only issues its share of the copies and meets the
            // barriers.
            const int hlast = (min(kv_end - 1, vis_max) >> 5);
            // The copies of tile step t: K(t+3) into the buffer of K(t), V(t+2)
            // into that of V(t-1).
            auto copy_ahead = [&](int t, LDS3 char *kload, LDS3 char *vload)
                                  __attribute__((always_inline)) {
                const E *kbase = Kh + (size_t)(t + 3) * kBc * kn;
                const E *vbase = Vh + (size_t)(t + 2) * kBc * vn;
                const int krows = min(kBc, kv_end - (t + 3) * kBc);
                const int vrows = min(kBc, kv_end - (t + 2) * kBc);
#pragma unroll
                for (int u = 0; u < kLoads; ++u) {
                    tile_load<D, W, STRIDED>(kbase, krows, kn, kload, k_src, u, wave);
                    tile_load<D, W, STRIDED>(vbase, vrows, vn, vload, v_src, u, wave);
                }
            };
            auto tile_step = [&](int t, int b) __attribute__((always_inline)) {
                const int b1 = (b + 1) % 3, b2 = (b + 2) % 3;
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if constexpr (kSafeSync) {
                    // Checking build: the copies land and are visible before
                    // the tile step computes.
                    copy_ahead(t, kb[b], vb[b2]);
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
                    step(2 * t + 1, no_loads, kb[b1], 0, vb[b], 0, kb[b1], 1, vb[b], 1, kb[b], vb[b2],
                         vf0, kf0, sB, sA, pA, pB);
                } else {
                    step(2 * t + 1, with_loads, kb[b1], 0, vb[b], 0, kb[b1], 1, vb[b], 1, kb[b], vb[b2],
                         vf0, kf0, sB, sA, pA, pB);
                }
                step(2 * t + 2, no_loads, kb[b1], 1, vb[b], 1, kb[b2], 0, vb[b1], 0, kb[b], vb[b2], vf0,
                     kf0, sA, sB, pB, pA);
            };
            int t = 0;
            for (; t < n_tiles; t += 3) {
                if (2 * t + 1 > hlast + 1) break;
                tile_step(t, 0);
                if (t + 1 >= n_tiles) {
                    t += 1;
                    break;
                }
                if (2 * t + 3 > hlast + 1) {
                    t += 1;
                    break;
                }
                tile_step(t + 1, 1);
                if (t + 2 >= n_tiles) {
                    t += 2;
                    break;
                }
                if (2 * t + 5 > hlast + 1) {
                    t += 2;
                    break;
                }
                tile_step(t + 2, 2);
            }
            for (; t < n_tiles; ++t) {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                const int b = t % 3;
                LDS3 char *kload = b == 0 ? kb[0] : b == 1 ? kb[1] : kb[2];
                LDS3 char *vload = b == 0 ? vb[2] : b == 1 ? vb[0] : vb[1];
                copy_ahead(t, kload, vload);
                if constexpr (kSafeSync) {  // the second barrier of a checking tile step
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
                }
            }

            // O = acc / (sum of the rounded probabilities) rounded to the element
            // type; LSE = m * scale + ln(l) with the fp32 sum l.
            float l_tot;
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                                 __float_as_uint(l_run), false, false);
                l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            const float inv = 1.f / lr_run;
            if (qrow < N) {
                E *orow = O + ooff + (size_t)qrow * on;
        #pragma unroll
                for (int db = 0; db < DB; ++db)
        #pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        f32x4 x;
        #pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * a + e] * inv;
                        *reinterpret_cast<X4 *>(orow + 32 * db + 8 * a + 4 * g) =
                            __builtin_convertvector(x, X4);
                    }
                if (g == 0) LSE[(size_t)bh * N + qrow] = m_run * scale + logf(l_tot);
            }
        }
    }
}

// Head dim 128 takes the software-pipelined kernel with 8-wave workgroups
// (256 query rows).  Causal head dim 64 with long sequences (N >= 8192)
// takes it with 4-wave workgroups (two per CU); there it measured 3-4 %
// faster than the 128-row kernel, which stays ahead on shorter sequences
// (fewer, longer workgroups start and drain less evenly).  The other head
// dims (every multiple of 16 up to 128) take the 128-row kernel.
constexpr int kPipeWaves = 8;
constexpr int kPipeWaves64 = 4;
constexpr int kPipeMinN64 = 8192;

// Schedule of a forward launch with `slots` persistent workgroup slots (see
// sched_item): mode 2 when the heads and slots split evenly over the XCDs and,
// under the causal mask, the rounds pair up; tile pairs (mode 1) when there
// are enough of them to balance; otherwise one workgroup per tile (mode 3).
void plan_forward(bool causal, int n_bh, int nqt, long slots, int &mode, long &grid) {
    const long n_tiles = (long)n_bh * nqt;
    mode = 3;
    grid = n_tiles;
    if (n_tiles < slots || slots % 8 != 0) return;
    if (n_bh % 8 == 0) {
        const long L = slots / 8, n_local = (long)(n_bh / 8) * nqt;
        const long rounds = (n_local + L - 1) / L;
        if (!causal || (n_local % L == 0 && rounds % 2 == 0)) {
            mode = 2;
            grid = slots;
            return;
        }
    }
    const long n_pairs = (long)n_bh * ((nqt + 1) / 2);
    if (causal && n_pairs >= slots && (n_pairs % slots == 0 || n_pairs >= 4 * slots)) {
        mode = 1;
        grid = slots;
    }
}

// True when `tiles` workgroups fill the slots of three workgroups per
// compute unit at least as evenly as those of two (the last round's share
// of occupied slots).
bool fills_as_evenly(long tiles, int cus) {
    const long s2 = 2L * cus, s3 = 3L * cus;
    const long r2 = (tiles + s2 - 1) / s2, r3 = (tiles + s3 - 1) / s3;
    return r3 * s3 <= r2 * s2;
}

// The launch of fwd_pipe_kernel.  W = 8 (96 KiB of LDS, one workgroup per
// compute unit): persistent, one workgroup per compute unit, at most one per
// work unit (modes 0-2).  W = 4: one workgroup per tile (mode 3); the
// persistent form measured 6 % slower there (B1 H16 N16384 d64 causal, same
// box), as two workgroups of one wave per SIMD share a compute unit and run
// unequal tiles side by side.
template <typename E, int D, bool CAUSAL, bool STRIDED, int W>
hipError_t launch_pipe(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                       int H, int N, float scale, float scale_log2, const FwdStrides &st,
                       hipStream_t stream) {
    constexpr int kRows = W * kRowsPerWave;
    const int nqt = (N + kRows - 1) / kRows;
    const int n_bh = B * H;
    int mode = 3;
    long grid = (long)n_bh * nqt;
    if (W == 8) plan_forward(CAUSAL, n_bh, nqt, device_cus(), mode, grid);
    hipLaunchKernelGGL((fwd_pipe_kernel<E, D, CAUSAL, STRIDED, W>), dim3((int)grid), dim3(64 * W),
                       0, stream, static_cast<const E *>(q), static_cast<const E *>(k),
                       static_cast<const E *>(v), static_cast<E *>(o), lse, N, nqt, n_bh, mode,
                       scale, scale_log2, st);
    return hipGetLastError();
}

template <typename E, int D, bool CAUSAL, bool STRIDED>
hipError_t launch(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                  int N, float scale, const FwdStrides &st, hipStream_t stream) {
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    if constexpr (D == 128) {
        return launch_pipe<E, D, CAUSAL, STRIDED, kPipeWaves>(q, k, v, o, lse, B, H, N, scale,
                                                              scale_log2, st, stream);
    } else {
        if constexpr (D == 64 && CAUSAL) {
            if (N >= kPipeMinN64)
                return launch_pipe<E, D, CAUSAL, STRIDED, kPipeWaves64>(q, k, v, o, lse, B, H, N,
                                                                        scale, scale_log2, st,
                                                                        stream);
        }
        // One workgroup per tile (mode 3).  The persistent schedules
        // (two workgroups per compute unit) measured slower here, same box:
        // B16 H12 N1000 d64 651 vs 700 TFLOP/s non-causal, 502 vs 529 causal,
        // B4 H16 N2048 d64 level; with rows this short a workgroup's
        // prologue (Q load, first tiles) is a large share of its time, and
        // other workgroups on the unit cover it only under the dispatcher.
        const int nqt = (N + kBr - 1) / kBr;
        const int n_bh = B * H;
        if constexpr (D == 64) {
            // Three workgroups per compute unit (a few registers go to
            // scratch) when the grid fills three slots per unit as evenly as
            // two, or under the causal mask, where the largest-first order
            // balances uneven workgroups: B16 H12 N1000 d64 +4 % causal, +5 %
            // non-causal; B4 H16 N2048 d64 (two full rounds of two, 1.33 of
            // three) 3 % slower, so it keeps two.
            if (CAUSAL || fills_as_evenly((long)n_bh * nqt, device_cus())) {
                hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, STRIDED, 3>), dim3(n_bh * nqt),
                                   dim3(kThreads), 0, stream, static_cast<const E *>(q),
                                   static_cast<const E *>(k), static_cast<const E *>(v),
                                   static_cast<E *>(o), lse, N, nqt, n_bh, 3, scale, scale_log2, st);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, STRIDED>), dim3(n_bh * nqt), dim3(kThreads),
                           0, stream, static_cast<const E *>(q), static_cast<const E *>(k),
                           static_cast<const E *>(v), static_cast<E *>(o), lse, N, nqt, n_bh, 3,
                           scale, scale_log2, st);
    }
    return hipGetLastError();
}

template <typename E, int D, bool STRIDED>
hipError_t launch_c(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                    int N, float scale, bool causal, const FwdStrides &st, hipStream_t stream) {
    return causal ? launch<E, D, true, STRIDED>(q, k, v, o, lse, B, H, N, scale, st, stream)
                  : launch<E, D, false, STRIDED>(q, k, v, o, lse, B, H, N, scale, st, stream);
}

template <typename E, bool STRIDED>
hipError_t launch_e(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                    int N, int d, float scale, bool causal, const FwdStrides &st,
                    hipStream_t stream) {
#define FA_FWD_CASE(DH) \
    case DH: return launch_c<E, DH, STRIDED>(q, k, v, o, lse, B, H, N, scale, causal, st, stream)
    switch (d) {
        FA_FWD_CASE(16);
        FA_FWD_CASE(32);
        FA_FWD_CASE(48);
        FA_FWD_CASE(64);
        FA_FWD_CASE(80);
        FA_FWD_CASE(96);
        FA_FWD_CASE(112);
        default: return launch_c<E, 128, STRIDED>(q, k, v, o, lse, B, H, N, scale, causal, st, stream);
    }
#undef FA_FWD_CASE
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream) {
    const FwdStrides none = {};
    return launch_e<__bf16, false>(q, k, v, o, lse, B, H, N, d, scale, causal, none, stream);
}

hipError_t launch_fwd_ex(bool fp16, const void *q, const void *k, const void *v, void *o,
                         float *lse, int B, int H, int N, int d, float scale, bool causal,
                         const int64_t *strides, hipStream_t stream) {
    const int64_t *sq = strides, *sk = strides + 3, *sv = strides + 6, *so = strides + 9;
    const long long hd = (long long)N * d, bd = (long long)H * hd;
    bool dense = true;
    for (const int64_t *t : {sq, sk, sv, so}) dense = dense && t[0] == bd && t[1] == hd && t[2] == d;
    FwdStrides st;
    st.qb = sq[0]; st.qh = sq[1]; st.qn = (int)sq[2];
    st.kb = sk[0]; st.kh = sk[1]; st.kn = (int)sk[2];
    st.vb = sv[0]; st.vh = sv[1]; st.vn = (int)sv[2];
    st.ob = so[0]; st.oh = so[1]; st.on = (int)so[2];
    st.H = H;
    if (fp16)
        return dense ? launch_e<_Float16, false>(q, k, v, o, lse, B, H, N, d, scale, causal, st, stream)
                     : launch_e<_Float16, true>(q, k, v, o, lse, B, H, N, d, scale, causal, st, stream);
    return dense ? launch_e<__bf16, false>(q, k, v, o, lse, B, H, N, d, scale, causal, st, stream)
                 : launch_e<__bf16, true>(q, k, v, o, lse, B, H, N, d, scale, causal, st, stream);
}

}  // namespace fa
