// fa_api.cpp -- the C ABI of libfa (declared in include/fa.h): argument
// validation, kernel selection and launch.  Every check runs before anything
// is enqueued; no HIP runtime call is made for an invalid argument list.
#include "fa.h"

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fa_internal.h"

namespace {

bool overlaps(const void *a, uint64_t a_bytes, const void *b, uint64_t b_bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}

// Head dims of every entry point: multiples of 16 from 16 to 128.
bool head_dim_ok(int d) { return d >= 16 && d <= 128 && d % 16 == 0; }

// Launch-size limit: at most 2^22 (batch*head, 128-row block) pairs, so that
// no kernel of a call launches 2^31 or more work-items (the largest grid,
// 512 threads per 256 rows, stays within 2^31) and every workgroup count fits
// an int.  Decode adds the same bound on its B*H*Nq output rows (one
// 256-thread merge workgroup each).
constexpr uint64_t kMaxRowBlocks = 1ull << 22;
bool grid_ok(int B, int H, int N) {
    return (uint64_t)B * (uint64_t)H * (((uint64_t)N + 127) / 128) <= kMaxRowBlocks;
}

int validate(const void *q, const void *k, const void *v, const void *o, const void *lse,
             int B, int H, int N, int d, float scale, uint64_t elem_bytes) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || N > (1 << 30)) return FA_ERR_SHAPE;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    // B*H*N*d < 2^40, evaluated without overflow (N*d < 2^38, B*H < 2^62).
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    if (bh > ((1ull << 40) - 1) / ((uint64_t)N * (uint64_t)d)) return FA_ERR_SHAPE;
    if (!grid_ok(B, H, N)) return FA_ERR_SHAPE;
    const uint64_t rows = bh * (uint64_t)N;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    for (const void *p : {q, k, v, o, lse})
        if (reinterpret_cast<uintptr_t>(p) & 15u) return FA_ERR_ALIGN;
    const uint64_t t_bytes = rows * (uint64_t)d * elem_bytes;
    const uint64_t l_bytes = rows * 4u;
    for (const void *in : {q, k, v}) {
        if (overlaps(o, t_bytes, in, t_bytes)) return FA_ERR_ALIAS;
        if (overlaps(lse, l_bytes, in, t_bytes)) return FA_ERR_ALIAS;
    }
    if (overlaps(o, t_bytes, lse, l_bytes)) return FA_ERR_ALIAS;
    return FA_OK;
}

// fa_bwd: the shared checks of `validate` on the forward quantities, then
// the extra pointers and their aliasing.
int validate_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const void *lse, const void *dq, const void *dk, const void *dv,
                 const void *delta, int B, int H, int N, int d, float scale) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || N > (1 << 30)) return FA_ERR_SHAPE;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    if (bh > ((1ull << 40) - 1) / ((uint64_t)N * (uint64_t)d)) return FA_ERR_SHAPE;
    if (!grid_ok(B, H, N)) return FA_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    for (const void *p : {q, k, v, o, dout, lse, dq, dk, dv, delta})
        if (reinterpret_cast<uintptr_t>(p) & 15u) return FA_ERR_ALIGN;
    const uint64_t rows = bh * (uint64_t)N;
    const uint64_t t_bytes = rows * (uint64_t)d * 2u;
    const uint64_t l_bytes = rows * 4u;
    struct Span { const void *p; uint64_t n; };
    const Span ins[] = {{q, t_bytes}, {k, t_bytes}, {v, t_bytes}, {o, t_bytes},
                        {dout, t_bytes}, {lse, l_bytes}};
    const Span outs[] = {{dq, t_bytes}, {dk, t_bytes}, {dv, t_bytes}, {delta, l_bytes}};
    for (const Span &w : outs)
        for (const Span &r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_ALIAS;
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return FA_ERR_ALIAS;
    return FA_OK;
}

bool decode_shape_ok(int B, int H, int Nq, int Nk, int d) {
    if (B < 1 || H < 1 || Nq < 1 || Nq > fa::kDecodeMaxQueries || Nk < Nq || Nk > (1 << 30))
        return false;
    if (!head_dim_ok(d)) return false;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    if (bh * (uint64_t)Nq > kMaxRowBlocks || !grid_ok(B, H, Nk)) return false;
    return bh <= ((1ull << 40) - 1) / ((uint64_t)Nk * (uint64_t)d);
}

// Partial outputs [B,H,S,Nq,d] then partial LSEs [B,H,S,Nq], fp32.
uint64_t decode_workspace(int B, int H, int Nq, int d, int S, uint64_t *lse_offset) {
    const uint64_t rows = (uint64_t)B * H * S * Nq;
    const uint64_t o_bytes = (rows * d * 4 + 255) / 256 * 256;
    if (lse_offset) *lse_offset = o_bytes;
    return o_bytes + rows * 4;
}

// O [B,H,N,d] then l, m [B,H,N], fp32, each part 256-byte aligned.
uint64_t kvouter_workspace(int B, int H, int N, int d, uint64_t *l_off, uint64_t *m_off) {
    const uint64_t rows = (uint64_t)B * H * N;
    const uint64_t o_bytes = (rows * d * 4 + 255) / 256 * 256;
    const uint64_t v_bytes = (rows * 4 + 255) / 256 * 256;
    if (l_off) *l_off = o_bytes;
    if (m_off) *m_off = o_bytes + v_bytes;
    return o_bytes + 2 * v_bytes;
}

bool shape_ok(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || N > (1 << 30)) return false;
    if (!head_dim_ok(d)) return false;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    return grid_ok(B, H, N) && bh <= ((1ull << 40) - 1) / ((uint64_t)N * (uint64_t)d);
}

// Byte span of a strided [B, H, N, d] view of 2-byte elements: one past the
// last byte any element occupies.
uint64_t view_span(const int64_t *s, int B, int H, int N, int d) {
    return ((uint64_t)(B - 1) * s[0] + (uint64_t)(H - 1) * s[1] + (uint64_t)(N - 1) * s[2] + d) * 2u;
}

// Rows of a strided view do not overlap: with the (extent > 1) dimensions
// sorted by stride, each stride reaches past everything the smaller ones
// cover (a row covers d elements).
bool rows_disjoint(const int64_t *s, int B, int H, int N, int d) {
    struct Dim { int64_t stride; int64_t extent; };
    Dim dims[3] = {{s[0], B}, {s[1], H}, {s[2], N}};
    std::sort(dims, dims + 3, [](const Dim &a, const Dim &b) { return a.stride < b.stride; });
    int64_t covered = d;  // elements spanned by the dimensions so far, from a row start
    for (const Dim &x : dims) {
        if (x.extent <= 1) continue;
        if (x.stride < covered) return false;
        covered = x.stride * (x.extent - 1) + covered;
    }
    return true;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
           int N, int d, float scale, int causal, hipStream_t stream) {
    const int rc = validate(q, k, v, o, lse, B, H, N, d, scale, 2);
    if (rc != FA_OK) return rc;
    const hipError_t e =
        fa::launch_fwd_bf16(q, k, v, o, lse, B, H, N, d, scale, causal != 0, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, int B,
               int H, int N, int d, float scale, int causal, hipStream_t stream) {
    const int rc = validate(q, k, v, o, lse, B, H, N, d, scale, 4);
    if (rc != FA_OK) return rc;
    const hipError_t e =
        fa::launch_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal != 0, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, float *delta, int B, int H, int N,
           int d, float scale, int causal, hipStream_t stream) {
    const int rc = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale);
    if (rc != FA_OK) return rc;
    const hipError_t e = fa::launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N,
                                             d, scale, causal != 0, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_ex(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int N, int d, float scale, int causal, const int64_t *strides,
              hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !strides) return FA_ERR_NULL;
    if (!shape_ok(B, H, N, d)) {
        if (B < 1 || H < 1 || N < 1 || N > (1 << 30)) return FA_ERR_SHAPE;
        if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
        return FA_ERR_SHAPE;
    }
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return FA_ERR_DTYPE;
    for (int t = 0; t < 4; ++t) {
        const int64_t *st = strides + 3 * t;
        if (st[0] < 0 || st[1] < 0 || st[2] < d || st[2] > (1 << 24)) return FA_ERR_STRIDE;
        if (st[0] > (int64_t)1 << 50 || st[1] > (int64_t)1 << 50) return FA_ERR_STRIDE;
    }
    for (const void *p : {q, k, v, (const void *)o, (const void *)lse})
        if (reinterpret_cast<uintptr_t>(p) & 15u) return FA_ERR_ALIGN;
    for (int t = 0; t < 12; ++t)
        if (strides[t] % 8) return FA_ERR_ALIGN;
    if (!rows_disjoint(strides + 9, B, H, N, d)) return FA_ERR_STRIDE;
    const uint64_t o_span = view_span(strides + 9, B, H, N, d);
    const uint64_t l_bytes = (uint64_t)B * H * N * 4u;
    const void *ins[3] = {q, k, v};
    for (int t = 0; t < 3; ++t) {
        const uint64_t span = view_span(strides + 3 * t, B, H, N, d);
        if (overlaps(o, o_span, ins[t], span) || overlaps(lse, l_bytes, ins[t], span))
            return FA_ERR_ALIAS;
    }
    if (overlaps(o, o_span, lse, l_bytes)) return FA_ERR_ALIAS;
    const hipError_t e = fa::launch_fwd_ex(dtype == FA_DTYPE_FP16, q, k, v, o, lse, B, H, N, d,
                                           scale, causal != 0,
                                           strides, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_ex(int dtype, const void *q, const void *k, const void *v, const void *o,
              const void *dout, const float *lse, void *dq, void *dk, void *dv, float *delta,
              int B, int H, int N, int d, float scale, int causal, const int64_t *strides,
              hipStream_t stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta || !strides)
        return FA_ERR_NULL;
    if (!shape_ok(B, H, N, d)) {
        if (B < 1 || H < 1 || N < 1 || N > (1 << 30)) return FA_ERR_SHAPE;
        if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
        return FA_ERR_SHAPE;
    }
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return FA_ERR_DTYPE;
    constexpr int kT = 8;  // q, k, v, o, dout, dq, dk, dv
    for (int t = 0; t < kT; ++t) {
        const int64_t *st = strides + 3 * t;
        if (st[0] < 0 || st[1] < 0 || st[2] < d || st[2] > (1 << 24)) return FA_ERR_STRIDE;
        if (st[0] > (int64_t)1 << 50 || st[1] > (int64_t)1 << 50) return FA_ERR_STRIDE;
    }
    for (const void *p : {q, k, v, o, dout, (const void *)lse, (const void *)dq, (const void *)dk,
                          (const void *)dv, (const void *)delta})
        if (reinterpret_cast<uintptr_t>(p) & 15u) return FA_ERR_ALIGN;
    for (int t = 0; t < 3 * kT; ++t)
        if (strides[t] % 8) return FA_ERR_ALIGN;
    for (int t = 5; t < kT; ++t)
        if (!rows_disjoint(strides + 3 * t, B, H, N, d)) return FA_ERR_STRIDE;
    const uint64_t l_bytes = (uint64_t)B * H * N * 4u;
    struct Span { const void *p; uint64_t n; };
    const Span ins[6] = {{q, view_span(strides + 0, B, H, N, d)},
                         {k, view_span(strides + 3, B, H, N, d)},
                         {v, view_span(strides + 6, B, H, N, d)},
                         {o, view_span(strides + 9, B, H, N, d)},
                         {dout, view_span(strides + 12, B, H, N, d)},
                         {lse, l_bytes}};
    const Span outs[4] = {{dq, view_span(strides + 15, B, H, N, d)},
                          {dk, view_span(strides + 18, B, H, N, d)},
                          {dv, view_span(strides + 21, B, H, N, d)},
                          {delta, l_bytes}};
    for (const Span &w : outs)
        for (const Span &r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_ALIAS;
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return FA_ERR_ALIAS;
    const hipError_t e = fa::launch_bwd_ex(dtype == FA_DTYPE_FP16, q, k, v, o, dout, lse, dq, dk,
                                           dv, delta, B, H, N, d, scale, causal != 0, strides,
                                           stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_kv_outer_workspace_size(int B, int H, int N, int d) {
    if (!shape_ok(B, H, N, d)) return 0;
    return (size_t)kvouter_workspace(B, H, N, d, nullptr, nullptr);
}

int fa_fwd_kv_outer(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                    int H, int N, int d, float scale, int causal, void *workspace,
                    size_t workspace_bytes, hipStream_t stream) {
    const int rc = validate(q, k, v, o, lse, B, H, N, d, scale, 2);
    if (rc != FA_OK) return rc;
    uint64_t l_off = 0, m_off = 0;
    const uint64_t need = kvouter_workspace(B, H, N, d, &l_off, &m_off);
    if (!workspace || (uint64_t)workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return FA_ERR_ALIGN;
    const uint64_t rows = (uint64_t)B * H * N;
    const uint64_t t_bytes = rows * d * 2;
    for (const void *p : {q, k, v, (const void *)o})
        if (overlaps(workspace, need, p, t_bytes)) return FA_ERR_ALIAS;
    if (overlaps(workspace, need, lse, rows * 4)) return FA_ERR_ALIAS;
    char *ws = static_cast<char *>(workspace);
    const hipError_t e = fa::launch_fwd_kvouter_bf16(
        q, k, v, o, lse, B, H, N, d, scale, causal != 0, reinterpret_cast<float *>(ws),
        reinterpret_cast<float *>(ws + l_off), reinterpret_cast<float *>(ws + m_off), stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits) {
    if (!decode_shape_ok(B, H, Nq, Nk, d)) return 0;
    const int S = fa::decode_num_splits(B, H, Nq, Nk, num_splits);
    return (size_t)decode_workspace(B, H, Nq, d, S, nullptr);
}

int fa_decode(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
              int Nq, int Nk, int d, float scale, int causal, int num_splits, void *workspace,
              size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 1 || Nq > fa::kDecodeMaxQueries || Nk < Nq || Nk > (1 << 30))
        return FA_ERR_SHAPE;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    if (!decode_shape_ok(B, H, Nq, Nk, d)) return FA_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    const int S = fa::decode_num_splits(B, H, Nq, Nk, num_splits);
    uint64_t lse_off = 0;
    const uint64_t need = decode_workspace(B, H, Nq, d, S, &lse_off);
    if (!workspace || (uint64_t)workspace_bytes < need) return FA_ERR_WORKSPACE;
    for (const void *p : {q, k, v, (const void *)o, (const void *)lse, (const void *)workspace})
        if (reinterpret_cast<uintptr_t>(p) & 15u) return FA_ERR_ALIGN;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    const uint64_t q_bytes = bh * Nq * d * 2, kv_bytes = bh * (uint64_t)Nk * d * 2;
    const uint64_t l_bytes = bh * Nq * 4;
    struct Span { const void *p; uint64_t n; };
    const Span ins[] = {{q, q_bytes}, {k, kv_bytes}, {v, kv_bytes}};
    const Span outs[] = {{o, q_bytes}, {lse, l_bytes}, {workspace, need}};
    for (const Span &w : outs)
        for (const Span &r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_ALIAS;
    for (int a = 0; a < 3; ++a)
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return FA_ERR_ALIAS;
    float *o_part = static_cast<float *>(workspace);
    float *lse_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + lse_off);
    const hipError_t e = fa::launch_decode_bf16(q, k, v, o, lse, B, H, Nq, Nk, d, scale,
                                                causal != 0, S, o_part, lse_part, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                      int H, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                      hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 1 || Nq > fa::kDecodeMaxQueries || Nk < Nq || Nk > (1 << 30))
        return FA_ERR_SHAPE;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    if (!decode_shape_ok(B, H, Nq, Nk, d)) return FA_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    const int S = fa::decode_num_splits(B, H, Nq, Nk, num_splits);
    uint64_t lse_off = 0;
    const uint64_t need = decode_workspace(B, H, Nq, d, S, &lse_off);
    if (need > fa::kDecodeScratchBytes) return FA_ERR_SCRATCH;
    for (const void *p : {q, k, v, (const void *)o, (const void *)lse})
        if (reinterpret_cast<uintptr_t>(p) & 15u) return FA_ERR_ALIGN;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    const uint64_t q_bytes = bh * Nq * d * 2, kv_bytes = bh * (uint64_t)Nk * d * 2;
    const uint64_t l_bytes = bh * Nq * 4;
    struct Span { const void *p; uint64_t n; };
    const Span ins[] = {{q, q_bytes}, {k, kv_bytes}, {v, kv_bytes}};
    const Span outs[] = {{o, q_bytes}, {lse, l_bytes}};
    for (const Span &w : outs)
        for (const Span &r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_ALIAS;
    if (overlaps(o, q_bytes, lse, l_bytes)) return FA_ERR_ALIAS;
    void *scratch = nullptr;
    if (fa::decode_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
    float *o_part = static_cast<float *>(scratch);
    float *lse_part = reinterpret_cast<float *>(static_cast<char *>(scratch) + lse_off);
    const hipError_t e = fa::launch_decode_bf16(q, k, v, o, lse, B, H, Nq, Nk, d, scale,
                                                causal != 0, S, o_part, lse_part, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_ex(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                 void *workspace, size_t workspace_bytes, const int64_t *strides,
                 hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !strides) return FA_ERR_NULL;
    if (B < 1 || H < 1 || Nq < 1 || Nq > fa::kDecodeMaxQueries || Nk < Nq || Nk > (1 << 30))
        return FA_ERR_SHAPE;
    if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
    if (!decode_shape_ok(B, H, Nq, Nk, d)) return FA_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return FA_ERR_DTYPE;
    for (int t = 0; t < 4; ++t) {
        const int64_t *st = strides + 3 * t;
        if (st[0] < 0 || st[1] < 0 || st[2] < d || st[2] > (1 << 24)) return FA_ERR_STRIDE;
        if (st[0] > (int64_t)1 << 50 || st[1] > (int64_t)1 << 50) return FA_ERR_STRIDE;
    }
    const int S = fa::decode_num_splits(B, H, Nq, Nk, num_splits);
    uint64_t lse_off = 0;
    const uint64_t need = decode_workspace(B, H, Nq, d, S, &lse_off);
    if (!workspace || (uint64_t)workspace_bytes < need) return FA_ERR_WORKSPACE;
    for (const void *p : {q, k, v, (const void *)o, (const void *)lse, (const void *)workspace})
        if (reinterpret_cast<uintptr_t>(p) & 15u) return FA_ERR_ALIGN;
    for (int t = 0; t < 12; ++t)
        if (strides[t] % 8) return FA_ERR_ALIGN;
    if (!rows_disjoint(strides + 9, B, H, Nq, d)) return FA_ERR_STRIDE;
    const uint64_t l_bytes = (uint64_t)B * H * Nq * 4;
    struct Span { const void *p; uint64_t n; };
    const Span ins[] = {{q, view_span(strides + 0, B, H, Nq, d)},
                        {k, view_span(strides + 3, B, H, Nk, d)},
                        {v, view_span(strides + 6, B, H, Nk, d)}};
    const Span outs[] = {{o, view_span(strides + 9, B, H, Nq, d)}, {lse, l_bytes},
                         {workspace, need}};
    for (const Span &w : outs)
        for (const Span &r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA_ERR_ALIAS;
    for (int a = 0; a < 3; ++a)
        for (int b = a + 1; b < 3; ++b)
            if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return FA_ERR_ALIAS;
    float *o_part = static_cast<float *>(workspace);
    float *lse_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + lse_off);
    const hipError_t e = fa::launch_decode_ex(dtype == FA_DTYPE_FP16, q, k, v, o, lse, B, H, Nq,
                                              Nk, d, scale, causal != 0, S, o_part, lse_part,
                                              strides, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char *fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "FA_OK: success";
        case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE: need B, H, N >= 1, N <= 2^30, B*H*N*d < 2^40 and B*H*ceil(N/128) <= 2^22";
        case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension d not supported (need a multiple of 16 from 16 to 128)";
        case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
        case FA_ERR_ALIGN: return "FA_ERR_ALIGN: every pointer must be 16-byte aligned";
        case FA_ERR_HIP: return "FA_ERR_HIP: the kernel launch failed";
        case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps an input or another output";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace is NULL or smaller than required";
        case FA_ERR_DTYPE: return "FA_ERR_DTYPE: dtype must be FA_DTYPE_BF16 or FA_DTYPE_FP16";
        case FA_ERR_STRIDE: return "FA_ERR_STRIDE: strides must be >= 0, row strides in [d, 2^24], output rows disjoint";
        case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: the partials of this call exceed the fixed scratch of fa_decode_noalloc (FA_DECODE_SCRATCH_BYTES); pass a smaller num_splits";
        default: return "unknown fa status code";
    }
}

}  // extern "C"
