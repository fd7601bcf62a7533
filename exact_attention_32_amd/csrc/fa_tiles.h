// fa_tiles.h -- device helpers shared by the kernels that stream 64-row
// tiles of a [N, d] bf16 or fp16 matrix through LDS with 256-thread
// workgroups and read them both row-wise (MFMA A operands of 32 x 16 blocks)
// and transposed (ds_read_b64_tr_b16): the swizzle, the direct-to-LDS tile
// copy, the lane read offsets, the element types' MFMA, and the store of a
// [d x 32] accumulator block as rows of the element type.
// Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

#define LDS3 __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;            // rows (queries or keys) owned by one wave
constexpr int kOuter = kWaves * kRowsPerWave;  // rows owned by one workgroup
constexpr int kInner = 64;                  // rows per streamed tile
constexpr float kLog2e = 1.4426950408889634f;

// Placed first in a block that runs under a uniform condition (a tile's
// element mask): an empty statement with side effects, so the optimiser
// cannot turn the block into selects that every tile would then execute.
__device__ __forceinline__ void keep_branch() { asm volatile("" ::: "memory"); }

// The same value, unknown to the optimiser at this point: what is derived
// from it is computed here, not hoisted and kept in registers from an
// earlier use (loop-invariant lane offsets under register pressure).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Marks a value as used at this point, so that the optimiser computes it
// before here (in this block) rather than next to its later use.
template <typename T>
__device__ __forceinline__ void pin(T &x) {
    asm volatile("" : "+v"(x));
}

// Operand vectors and the 32x32x16 MFMA (fp32 accumulation) of an element
// type.
template <typename E>
struct TileOps;
template <>
struct TileOps<__bf16> {
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
struct TileOps<_Float16> {
    typedef f16x8 x8;
    typedef f16x4 x4;
    static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// 0/1 selector for row sums of P^T operands on the matrix core: with it as
// the A operand of a 16 x 16 x 32 MFMA whose B operand is a P^T operand of
// O^T += V^T P^T (lane l: query l % 32, keys 8(l / 32) .. +7 of a 16-key
// step), every lane's four outputs hold the 16-key sum of its own query.  (The
// B operand is read as column l % 16, reduction index 8(l / 16) .. +7, so lane
// groups 0, 2 carry query n and groups 1, 3 query n + 16; row m selects
// reduction group k / 8 when (m / 4) and (k / 8) have the same parity, and the
// output lane l holds column l % 16, rows 4(l / 16) .. +3.)
template <typename E>
__device__ __forceinline__ typename TileOps<E>::x8 rowsum_selector(int lane) {
    typename TileOps<E>::x8 a;
    const float one = ((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1)) ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (E)one;
    return a;
}

// One swizzle for tiles read both by 128-bit row reads (16 rows x one 16-byte
// chunk per LDS pass) and by the 64-bit transpose read (4 rows x 4 chunks per
// pass): the stored chunk of logical chunk c in row r is c ^ swz(r).
//   d = 128 (one row per 256-byte line): swz = 4(r & 3) + ((r >> 2) & 3);
//   d = 64  (two rows per line):         swz = 4((r >> 1) & 1) + ((r >> 2) & 3).
// Both depend on r mod 16 only.
template <int D>
__device__ __forceinline__ int swz(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Workgroup id -> (batch*head, tile): consecutive ids go to consecutive XCDs.
// By default XCD x walks the contiguous range [x*W/8, (x+1)*W/8) of (head,
// tile) pairs when the grid divides evenly (its L2 then serves one head's
// stream).  With `by_cost` (causal: a tile's cost grows with its index, or
// falls with it when `reverse`) and fewer than `by_cost_below` tiles per
// head, ids go in order of decreasing cost, one cost rank after the other
// over all heads (largest first, so that cheap tiles fill the gaps at the
// end of the grid); with a head count that is a multiple of 8, id mod 8 =
// head mod 8, so every tile of a head still runs on one XCD.
__device__ __forceinline__ void map_block(int L, int W, int ntiles, bool reverse, bool by_cost,
                                          int by_cost_below, int &bh, int &tile) {
    if (by_cost && ntiles < by_cost_below) {
        const int heads = W / ntiles;
        const int rank = L / heads;
        bh = L - rank * heads;
        tile = reverse ? ntiles - 1 - rank : rank;
        return;
    }
    int gidx = L;
    if ((W & 7) == 0) gidx = (L & 7) * (W >> 3) + (L >> 3);
    bh = gidx / ntiles;
    tile = gidx - bh * ntiles;
    if (reverse) tile = ntiles - 1 - tile;
}

// Direct-to-LDS copy of one kInner-row tile of a [N, DH] matrix of 2-byte
// elements, rows `rs` elements apart (rows r0 .. r0 + kInner - 1; rows >= N
// read as zeros) into `dst`, a tile of kInner rows of D >= DH columns,
// swizzled: lane l of load u of wave w writes chunk position
// q = (u*kWaves + w)*64 + l, and fetches the logical chunk that the swizzle
// stores there.  Load u covers the rows 16 (D = 128) or 32 (D = 64) after
// load 0's, which leaves the row's swizzle term unchanged, so one lane
// offset `src` (load 0, tile_src_offset) serves every load, moved by that
// many rows.  The descriptor ends after the last valid row's DH elements.
// With DH < D the columns at and past DH receive copies of the same row's
// leading chunks (see tile_src_offset): callers use them only for output
// rows they never store.
template <int D, int DH = D, bool STRIDED = false>
__device__ __forceinline__ void load_tile(const void *mat, int N, int r0, LDS3 char *dst,
                                          uint32_t src, int wave, int rs = DH) {
    static_assert(DH <= D && DH % 16 == 0, "row length");
    constexpr int kLoads = kInner * (D / 8) / kThreads;
    constexpr int kRowsPerLoad = kWaves * 1024 / (D * 2);
    const int stride = STRIDED ? rs : DH;
    const uint32_t rows = (uint32_t)max(0, min(kInner, N - r0));
    // (readfirstlane: the clamp compiles to a vector med3, and a descriptor
    // in vector registers would be wrapped in a per-lane waterfall loop)
    const uint32_t bytes = __builtin_amdgcn_readfirstlane(
        STRIDED ? (rows ? (rows - 1) * (uint32_t)rs * 2u + DH * 2u : 0u) : rows * (uint32_t)(DH * 2));
    const __amdgpu_buffer_rsrc_t rsrc =
        make_rsrc((const char *)mat + (size_t)r0 * (size_t)stride * 2, bytes);
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc,
                                                 (LDS3 void *)(dst + (u * kWaves + wave) * 1024), 16,
                                                 src, u * kRowsPerLoad * stride * 2, 0, 0);
}

// Direct-to-LDS copy of vec[c0 .. c0 + 63] (fp32; entries at or past N read
// as 0) into dst[0 .. 63], one 4-byte load per lane of the calling wave.
__device__ __forceinline__ void load_vec(const float *vec, int N, int c0, LDS3 float *dst,
                                         int lane) {
    const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)max(0, min(kInner, N - c0)) * 4u);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(vec + c0, bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS3 void *)dst, 4, (uint32_t)lane * 4u, 0, 0, 0);
}

// Lane source offset of load_tile's first load (see there), rows `rs`
// elements apart.  A position whose logical chunk c lies at or past DH/8
// fetches chunk c mod DH/8 of the same row: every byte read belongs to a
// row of the matrix.
template <int D, int DH = D>
__device__ __forceinline__ uint32_t tile_src_offset(int wave, int lane, int rs = DH) {
    const int q = wave * 64 + lane;
    const int r = q / (D / 8);
    const int p = q % (D / 8);
    int c = p ^ swz<D>(r);
    if (DH < D) c %= DH / 8;
    return (uint32_t)(r * rs * 2 + (c << 4));
}

// Byte offset (within a tile) of the 128-bit operand read of k-step ks: lane
// (g, i) reads row i (+32 per 32-row block) and logical chunk 2ks + g.  The
// stored chunk is (2ks + g) ^ swz(i) = (g ^ swz(i)) ^ 2ks, so the offset is
// the k-step-0 offset with the chunk field XOR-ed by 32 ks bytes.
template <int D>
__device__ __forceinline__ uint32_t row_read_offset(int lane) {
    const int g = lane >> 5, i = lane & 31;
    return (uint32_t)(i * D * 2 + ((g ^ swz<D>(i)) << 4));
}
__device__ __forceinline__ uint32_t row_read_at(uint32_t base, int ks) {
    return base ^ (uint32_t)(ks << 5);
}

// Byte offsets of the transpose reads that form the A operand M^T (M = a
// tile, [row][d]) of a 32 (d) x 16 (rows) MFMA block: in 16-lane group
// G = lane/16 (m0 = 16 (G & 1), g = G >> 1), lane i of the group reads the
// four bf16 of row 16T + 8h + 4g + i/4, columns 32db + m0 + 4(i%4) .. +3; the
// two halves h = 0, 1 form one 8-element operand.  The swizzle term depends on
// h (not on T), so each h has its own offset; d-block db only adds 4db to
// the logical chunk, i.e. XORs the chunk field with 64 db bytes.
template <int D>
__device__ __forceinline__ void tr_read_offsets(int lane, uint32_t *off) {
    const int g = lane >> 5, gi = lane & 15, m0 = 16 * ((lane >> 4) & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + 4 * g + (gi >> 2);
        const int col = m0 + 4 * (gi & 3);
        const int c = col >> 3;
        off[h] = (uint32_t)(row * D * 2 + ((c ^ swz<D>(row)) << 4) + ((col & 4) << 1));
    }
}

template <int D, typename X8 = bf16x8>
__device__ __forceinline__ X8 tr_read(const LDS3 char *tile, const uint32_t *off, int T, int db) {
    const LDS3 char *base = tile + T * 16 * D * 2;
    const uint32_t x = (uint32_t)(db << 6);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 v4i16 *)(base + (off[0] ^ x)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS3 v4i16 *)(base + (off[1] ^ x)));
    return __builtin_bit_cast(X8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Store a [D x 32] accumulator block set (lane (g, j) holds row `row` of the
// result, columns 32db + 8a + 4g + e in acc[db][4a + e]) times `mul` as the
// element type E; only the first DH columns are stored.
template <int D, int DH = D, typename E = __bf16>
__device__ __forceinline__ void store_rows(E *row_ptr, const f32x16 *acc, float mul, int g) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            if (DH < D && 32 * db + 8 * a + 4 * g >= DH) continue;
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * a + e] * mul;
            typedef typename TileOps<E>::x4 X4;
            *reinterpret_cast<X4 *>(row_ptr + 32 * db + 8 * a + 4 * g) =
                __builtin_convertvector(x, X4);
        }
}

}  // namespace
}  // namespace fa
