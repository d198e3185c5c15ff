// C ABI of the attention library: argument validation on the host (before any
// HIP call), then one kernel launch on the caller's stream.  See include/sdpa.h
// for the contract of each entry point.
#include "sdpa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "sdpa_common.hpp"

namespace {

constexpr int kVersion = 1 * 10000 + 8 * 100 + 0;  // 1.8.0: dropout at widths 32 and 128

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [lo, lo + bytes) and [lo2, lo2 + bytes2) share a byte.
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Pointers, dtype, shapes, head widths, scale and base alignment (no aliasing).
int validate_core(const void* q, const void* k, const void* v, void* out, int32_t B, int32_t h,
                  int32_t n, int32_t m, int32_t d_k, int32_t d_v, float scale,
                  const int32_t* key_lens, int32_t dtype) {
    if (!q || !k || !v || !out) return SDPA_ERR_NULL;
    if (dtype != SDPA_F32 && dtype != SDPA_BF16) return SDPA_ERR_DTYPE;
    if (B < 1 || h < 1 || n < 1 || m < 1 || d_k < 1 || d_v < 1) return SDPA_ERR_SHAPE;
    // Element counts and the launch grid must stay well inside 64-bit offsets and
    // a 31-bit grid (blocks of at least 32 queries or keys per head):
    // B·h·max(n, m)·max(d) < 2^48 and B·h·⌈max(n, m)/32⌉ < 2^31.
    const uint64_t heads = (uint64_t)B * (uint64_t)h;
    const uint64_t rows = (uint64_t)(n > m ? n : m);
    const uint64_t width = (uint64_t)(d_k > d_v ? d_k : d_v);
    if (heads * rows * width >= (1ull << 48)) return SDPA_ERR_SHAPE;
    if (heads * ((rows + 31) / 32) >= (1ull << 31)) return SDPA_ERR_SHAPE;
    // The kernels address a head's rows with 32-bit byte offsets (buffer ranges
    // run from a tile to the end of its head): one head's Q, K, V or output
    // rows stay below 2 GiB.
    const uint64_t esz = dtype == SDPA_F32 ? 4 : 2;
    if (rows * width * esz >= (1ull << 31)) return SDPA_ERR_SHAPE;
    // Head widths: 64 and 64 for both dtypes; for bf16 also the pairs of
    // sdpa::width_supported (equal widths 16, 32, 128, 512; d_v = 64 with d_k = 16 or 32).
    const bool wide_ok = dtype == SDPA_BF16 && sdpa::width_supported(d_k, d_v);
    if (!(d_k == sdpa::kHeadDim && d_v == sdpa::kHeadDim) && !wide_ok) return SDPA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale) || !(scale > 0.f)) return SDPA_ERR_SCALE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SDPA_ERR_ALIGN;
    if (key_lens && (reinterpret_cast<uintptr_t>(key_lens) & 3u)) return SDPA_ERR_ALIGN;
    return SDPA_OK;
}

// Everything but the mask, for the packed [B, h, len, d] layout: validate_core
// and out overlapping none of q, k, v, key_lens.
int validate(const void* q, const void* k, const void* v, void* out, int32_t B, int32_t h,
             int32_t n, int32_t m, int32_t d_k, int32_t d_v, float scale,
             const int32_t* key_lens, int32_t dtype) {
    const int st = validate_core(q, k, v, out, B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    const uint64_t heads = (uint64_t)B * (uint64_t)h;
    const uint64_t esz = dtype == SDPA_F32 ? 4 : 2;
    const uint64_t qb = heads * n * d_k * esz, kb = heads * m * d_k * esz;
    const uint64_t vb = heads * m * d_v * esz, ob = heads * n * d_v * esz;
    if (overlap(out, ob, q, qb) || overlap(out, ob, k, kb) || overlap(out, ob, v, vb))
        return SDPA_ERR_ALIAS;
    if (key_lens && overlap(out, ob, key_lens, (uint64_t)B * sizeof(int32_t))) return SDPA_ERR_ALIAS;
    return SDPA_OK;
}

// Each launcher reports hipGetLastError after its launches.  That status is
// per thread and also holds errors of earlier, unrelated HIP calls that no one
// collected; it is cleared first so that SDPA_ERR_LAUNCH means this call's own
// launch was refused.
void clear_pending_error() { (void)hipGetLastError(); }

int launch(const sdpa::Args& a, int32_t dtype, void* stream) {
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    clear_pending_error();
    const hipError_t e = dtype == SDPA_BF16 ? sdpa::launch_bf16(a, s) : sdpa::launch_f32(a, s);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

}  // namespace

extern "C" int sdpa_forward(const void* q, const void* k, const void* v, void* out, int32_t B,
                            int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v, float scale,
                            int32_t mask_kind, const int32_t* key_lens, int32_t dtype,
                            void* stream) {
    const int st = validate(q, k, v, out, B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    if (mask_kind != SDPA_MASK_NONE && mask_kind != SDPA_MASK_CAUSAL) return SDPA_ERR_MASK;
    if (mask_kind == SDPA_MASK_CAUSAL && n != m) return SDPA_ERR_MASK;
    // causal = the window (unbounded, 0) at top-left alignment
    sdpa::Args a{q, k, v, out, B, h, n, m, scale, -1, mask_kind == SDPA_MASK_CAUSAL ? 0 : -1,
                 0, key_lens};
    a.d = d_k;
    a.dv = d_v;
    return launch(a, dtype, stream);
}

extern "C" int sdpa_forward_window(const void* q, const void* k, const void* v, void* out,
                                   int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k,
                                   int32_t d_v, float scale, int32_t window_left,
                                   int32_t window_right, int32_t align, const int32_t* key_lens,
                                   int32_t dtype, void* stream) {
    const int st = validate(q, k, v, out, B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    if (window_left < -1 || window_right < -1) return SDPA_ERR_MASK;
    if (align != SDPA_ALIGN_TOP_LEFT && align != SDPA_ALIGN_BOTTOM_RIGHT) return SDPA_ERR_MASK;
    // A side wider than n + m reaches past every key from every query: unbounded.
    const int64_t reach = (int64_t)n + m;
    const int32_t wl = window_left > reach ? -1 : window_left;
    const int32_t wr = window_right > reach ? -1 : window_right;
    sdpa::Args a{q, k, v, out, B, h, n, m, scale, wl, wr,
                 align == SDPA_ALIGN_BOTTOM_RIGHT ? 1 : 0, key_lens};
    a.d = d_k;
    a.dv = d_v;
    return launch(a, dtype, stream);
}

// Sublayer head widths: d_k = d_v ∈ {32, 64, 128}, with h·d a multiple of 64
// (the output projection contracts over h·d in steps of 64).
bool mha_width_ok(int32_t h, int32_t d_k, int32_t d_v) {
    if (d_k != d_v || (d_k != 32 && d_k != 64 && d_k != 128)) return false;
    return ((int64_t)h * d_k) % 64 == 0;
}

// Window arguments → (wl, wr, bottom_right), or SDPA_ERR_MASK.
int window_args(int32_t n, int32_t m, int32_t window_left, int32_t window_right, int32_t align,
                int32_t* wl, int32_t* wr, int32_t* br) {
    if (window_left < -1 || window_right < -1) return SDPA_ERR_MASK;
    if (align != SDPA_ALIGN_TOP_LEFT && align != SDPA_ALIGN_BOTTOM_RIGHT) return SDPA_ERR_MASK;
    // A side wider than n + m reaches past every key from every query: unbounded.
    const int64_t reach = (int64_t)n + m;
    *wl = window_left > reach ? -1 : window_left;
    *wr = window_right > reach ? -1 : window_right;
    *br = align == SDPA_ALIGN_BOTTOM_RIGHT ? 1 : 0;
    return SDPA_OK;
}

extern "C" int sdpa_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse,
                                int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                                float scale, int32_t window_left, int32_t window_right,
                                int32_t align, const int32_t* key_lens, int32_t dtype, void* stream) {
    int st = validate(q, k, v, out, B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    if (!lse) return SDPA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return SDPA_ERR_ALIGN;
    int32_t wl, wr, br;
    st = window_args(n, m, window_left, window_right, align, &wl, &wr, &br);
    if (st != SDPA_OK) return st;
    const uint64_t heads = (uint64_t)B * h;
    const uint64_t lb = heads * n * 4;
    const uint64_t esz = dtype == SDPA_F32 ? 4 : 2;
    const struct { const void* p; uint64_t n; } bufs[] = {
        {q, heads * n * d_k * esz}, {k, heads * m * d_k * esz}, {v, heads * m * d_v * esz},
        {out, heads * n * d_v * esz}, {key_lens, key_lens ? (uint64_t)B * 4 : 0}};
    for (const auto& b : bufs)
        if (b.p && overlap(lse, lb, b.p, b.n)) return SDPA_ERR_ALIAS;
    sdpa::Args a{q, k, v, out, B, h, n, m, scale, wl, wr, br, key_lens};
    a.lse = lse;
    a.d = d_k;
    a.dv = d_v;
    return launch(a, dtype, stream);
}

size_t forward_work_bytes(int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                          int32_t dtype) {
    if (B < 1 || h < 1 || n < 1 || m < 1 || dtype != SDPA_BF16) return 0;
    if (d_k != sdpa::kHeadDim || d_v != sdpa::kHeadDim) return 0;
    sdpa::Args a{nullptr, nullptr, nullptr, nullptr, B, h, n, m, 1.f, -1, -1, 0, nullptr};
    if (sdpa::short_bf16_fits(a)) return 0;
    return sdpa::decode_split_bytes(B, h, n, m);
}

extern "C" size_t sdpa_forward_workspace_bytes(int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k,
                                               int32_t d_v, int32_t dtype) {
    return forward_work_bytes(B, h, n, m, d_k, d_v, dtype);
}

extern "C" int sdpa_forward_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                               int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                               float scale, int32_t window_left, int32_t window_right, int32_t align,
                               const int32_t* key_lens, int32_t dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
    int st = validate(q, k, v, out, B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    int32_t wl, wr, br;
    st = window_args(n, m, window_left, window_right, align, &wl, &wr, &br);
    if (st != SDPA_OK) return st;
    const uint64_t heads = (uint64_t)B * h;
    struct Buf { const void* p; uint64_t n; };
    const Buf ins[] = {{q, heads * n * d_k * (dtype == SDPA_F32 ? 4 : 2)},
                       {k, heads * m * d_k * (dtype == SDPA_F32 ? 4 : 2)},
                       {v, heads * m * d_v * (dtype == SDPA_F32 ? 4 : 2)},
                       {out, heads * n * d_v * (dtype == SDPA_F32 ? 4 : 2)},
                       {key_lens, key_lens ? (uint64_t)B * 4 : 0}};
    if (lse) {
        if (reinterpret_cast<uintptr_t>(lse) & 3u) return SDPA_ERR_ALIGN;
        for (const Buf& b : ins)
            if (b.p && overlap(lse, heads * n * 4, b.p, b.n)) return SDPA_ERR_ALIAS;
    }
    const size_t need = forward_work_bytes(B, h, n, m, d_k, d_v, dtype);
    void* work = nullptr;
    if (workspace && need > 0) {
        if (!aligned16(workspace)) return SDPA_ERR_ALIGN;
        if (workspace_bytes < need) return SDPA_ERR_WORKSPACE;
        for (const Buf& b : ins)
            if (b.p && overlap(workspace, need, b.p, b.n)) return SDPA_ERR_ALIAS;
        if (lse && overlap(workspace, need, lse, heads * n * 4)) return SDPA_ERR_ALIAS;
        work = workspace;
    }
    sdpa::Args a{q, k, v, out, B, h, n, m, scale, wl, wr, br, key_lens};
    a.lse = lse;
    a.d = d_k;
    a.dv = d_v;
    a.work = work;
    a.work_bytes = work ? workspace_bytes : 0;
    return launch(a, dtype, stream);
}

extern "C" size_t sdpa_backward_workspace_bytes(int32_t B, int32_t h, int32_t n) {
    if (B < 1 || h < 1 || n < 1) return 0;
    return sdpa::bwd_workspace_bytes(B, h, n);
}

namespace {

// Keep-bit words of attention dropout: [B, h, n, ⌈m/32⌉] uint32.
uint64_t keep_bytes(int32_t B, int32_t h, int32_t n, int32_t m) {
    return (uint64_t)B * h * n * (((uint64_t)m + 31) / 32) * 4;
}

// The mask, its factor and the widths the dropout kernels take.
int validate_dropout(const uint32_t* keep, float keep_scale, int32_t d_k, int32_t d_v, int32_t dtype) {
    if (!keep) return SDPA_ERR_NULL;
    if (dtype != SDPA_BF16 || d_k != d_v || (d_k != 32 && d_k != 64 && d_k != 128)) return SDPA_ERR_UNSUPPORTED;
    if (!std::isfinite(keep_scale) || !(keep_scale > 0.f)) return SDPA_ERR_SCALE;
    if (reinterpret_cast<uintptr_t>(keep) & 3u) return SDPA_ERR_ALIGN;
    return SDPA_OK;
}

int backward_impl(const void* q, const void* k, const void* v, const void* out, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int32_t B, int32_t h, int32_t n,
                  int32_t m, int32_t d_k, int32_t d_v, float scale, int32_t window_left,
                  int32_t window_right, int32_t align, const int32_t* key_lens, const uint32_t* keep,
                  float keep_scale, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (!dout || !lse || !dq || !dk || !dv || !workspace) return SDPA_ERR_NULL;
    // q, k, v, out, shapes, scale, key_lens (out is an input here: the alias
    // checks below cover the outputs).
    int st = validate(q, k, v, const_cast<void*>(out), B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    // The bf16 backward kernels take equal widths 32, 64 and 128; the fp32 ones 64.
    if (d_k != d_v || (d_k != 32 && d_k != 64 && d_k != 128)) return SDPA_ERR_UNSUPPORTED;
    if (dtype == SDPA_F32 && d_k != sdpa::kHeadDim) return SDPA_ERR_UNSUPPORTED;
    for (const void* p : {dout, (const void*)dq, (const void*)dk, (const void*)dv, (const void*)workspace})
        if (!aligned16(p)) return SDPA_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return SDPA_ERR_ALIGN;
    int32_t wl, wr, br;
    st = window_args(n, m, window_left, window_right, align, &wl, &wr, &br);
    if (st != SDPA_OK) return st;
    const size_t need = sdpa::bwd_workspace_bytes(B, h, n);
    if (workspace_bytes < need) return SDPA_ERR_WORKSPACE;
    const uint64_t heads = (uint64_t)B * h, esz = dtype == SDPA_F32 ? 4 : 2;
    struct Buf { const void* p; uint64_t n; };
    const Buf ins[] = {{q, heads * n * d_k * esz}, {k, heads * m * d_k * esz}, {v, heads * m * d_v * esz},
                       {out, heads * n * d_v * esz}, {dout, heads * n * d_v * esz}, {lse, heads * n * 4},
                       {key_lens, key_lens ? (uint64_t)B * 4 : 0},
                       {keep, keep ? keep_bytes(B, h, n, m) : 0}};
    const Buf outs[] = {{dq, heads * n * d_k * esz}, {dk, heads * m * d_k * esz}, {dv, heads * m * d_v * esz},
                        {workspace, need}};
    for (int i = 0; i < 4; ++i) {
        for (const Buf& in : ins)
            if (in.p && overlap(outs[i].p, outs[i].n, in.p, in.n)) return SDPA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return SDPA_ERR_ALIAS;
    }
    sdpa::BwdArgs a{q, k, v, out, dout, lse, dq, dk, dv, workspace, B, h, n, m, scale, wl, wr, br,
                    key_lens, d_k};
    a.keep = keep;
    a.keep_scale = keep_scale;
    clear_pending_error();
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = dtype == SDPA_F32 ? sdpa::launch_bwd_f32(a, s) : sdpa::launch_bwd_bf16(a, s);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

}  // namespace

extern "C" int sdpa_backward(const void* q, const void* k, const void* v, const void* out,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                             float scale, int32_t window_left, int32_t window_right, int32_t align,
                             const int32_t* key_lens, int32_t dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return backward_impl(q, k, v, out, dout, lse, dq, dk, dv, B, h, n, m, d_k, d_v, scale, window_left,
                         window_right, align, key_lens, nullptr, 1.f, dtype, workspace, workspace_bytes,
                         stream);
}

extern "C" int sdpa_forward_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                                    int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                                    float scale, int32_t window_left, int32_t window_right, int32_t align,
                                    const int32_t* key_lens, const uint32_t* keep_mask, float keep_scale,
                                    int32_t dtype, void* stream) {
    int st = validate(q, k, v, out, B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    if ((st = validate_dropout(keep_mask, keep_scale, d_k, d_v, dtype)) != SDPA_OK) return st;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return SDPA_ERR_ALIGN;
    int32_t wl, wr, br;
    st = window_args(n, m, window_left, window_right, align, &wl, &wr, &br);
    if (st != SDPA_OK) return st;
    const uint64_t heads = (uint64_t)B * h;
    const uint64_t ob = heads * n * d_v * 2, lb = heads * n * 4, kb = keep_bytes(B, h, n, m);
    if (overlap(out, ob, keep_mask, kb)) return SDPA_ERR_ALIAS;
    if (lse) {
        const struct { const void* p; uint64_t n; } bufs[] = {
            {q, heads * n * d_k * 2}, {k, heads * m * d_k * 2}, {v, heads * m * d_v * 2},
            {out, ob}, {key_lens, key_lens ? (uint64_t)B * 4 : 0}, {keep_mask, kb}};
        for (const auto& b : bufs)
            if (b.p && overlap(lse, lb, b.p, b.n)) return SDPA_ERR_ALIAS;
    }
    sdpa::Args a{q, k, v, out, B, h, n, m, scale, wl, wr, br, key_lens};
    a.lse = lse;
    a.d = d_k;
    a.dv = d_v;
    a.keep = keep_mask;
    a.keep_scale = keep_scale;
    return launch(a, dtype, stream);
}

extern "C" int sdpa_backward_dropout(const void* q, const void* k, const void* v, const void* out,
                                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                     int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k, int32_t d_v,
                                     float scale, int32_t window_left, int32_t window_right, int32_t align,
                                     const int32_t* key_lens, const uint32_t* keep_mask, float keep_scale,
                                     int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != SDPA_F32 && dtype != SDPA_BF16) return SDPA_ERR_DTYPE;
    const int st = validate_dropout(keep_mask, keep_scale, d_k, d_v, dtype);
    if (st != SDPA_OK) return st;
    return backward_impl(q, k, v, out, dout, lse, dq, dk, dv, B, h, n, m, d_k, d_v, scale, window_left,
                         window_right, align, key_lens, keep_mask, keep_scale, dtype, workspace,
                         workspace_bytes, stream);
}

extern "C" size_t sdpa_mha_workspace_bytes(int32_t B, int32_t n, int32_t m, int32_t h, int32_t d_k,
                                           int32_t d_v) {
    if (B < 1 || n < 1 || m < 1 || h < 1 || !mha_width_ok(h, d_k, d_v)) return 0;
    return sdpa::mha_workspace_bytes(B, n, m, h, d_k);
}

extern "C" int sdpa_mha_forward(const void* x_q, const void* x_kv, const void* w_q, const void* w_k,
                                const void* w_v, const void* w_o, void* out, int32_t B, int32_t n,
                                int32_t m, int32_t d_model, int32_t h, int32_t d_k, int32_t d_v,
                                float scale, int32_t window_left, int32_t window_right,
                                int32_t align, const int32_t* key_lens, int32_t dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (!x_q || !x_kv || !w_q || !w_k || !w_v || !w_o || !out || !workspace) return SDPA_ERR_NULL;
    if (dtype != SDPA_F32 && dtype != SDPA_BF16) return SDPA_ERR_DTYPE;
    if (B < 1 || n < 1 || m < 1 || d_model < 1 || h < 1 || d_k < 1 || d_v < 1) return SDPA_ERR_SHAPE;
    if (dtype != SDPA_BF16 || !mha_width_ok(h, d_k, d_v) || d_model % 64 != 0) return SDPA_ERR_UNSUPPORTED;
    // Byte sizes; the kernels index with 32-bit offsets, so each stays below 2^31.
    const uint64_t lim = 1ull << 31;
    const uint64_t xq_b = (uint64_t)B * n * d_model * 2, xkv_b = (uint64_t)B * m * d_model * 2;
    const uint64_t w_b = (uint64_t)h * d_k * d_model * 2;
    const uint64_t need = sdpa::mha_workspace_bytes(B, n, m, h, d_k);
    if (xq_b >= lim || xkv_b >= lim || w_b >= lim || need >= lim) return SDPA_ERR_SHAPE;
    if ((uint64_t)B * h * (((uint64_t)n + 31) / 32) >= lim) return SDPA_ERR_SHAPE;
    if (window_left < -1 || window_right < -1) return SDPA_ERR_MASK;
    if (align != SDPA_ALIGN_TOP_LEFT && align != SDPA_ALIGN_BOTTOM_RIGHT) return SDPA_ERR_MASK;
    if (!std::isfinite(scale) || !(scale > 0.f)) return SDPA_ERR_SCALE;
    for (const void* p : {x_q, x_kv, w_q, w_k, w_v, w_o, (const void*)out, (const void*)workspace})
        if (!aligned16(p)) return SDPA_ERR_ALIGN;
    if (key_lens && (reinterpret_cast<uintptr_t>(key_lens) & 3u)) return SDPA_ERR_ALIGN;
    if (workspace_bytes < need) return SDPA_ERR_WORKSPACE;
    const uint64_t out_b = xq_b;
    struct Buf { const void* p; uint64_t n; };
    const Buf inputs[] = {{x_q, xq_b}, {x_kv, xkv_b}, {w_q, w_b}, {w_k, w_b}, {w_v, w_b}, {w_o, w_b},
                          {key_lens, key_lens ? (uint64_t)B * 4 : 0}};
    for (const Buf& in : inputs) {
        if (in.p && overlap(out, out_b, in.p, in.n)) return SDPA_ERR_ALIAS;
        if (in.p && overlap(workspace, need, in.p, in.n)) return SDPA_ERR_ALIAS;
    }
    if (overlap(out, out_b, workspace, need)) return SDPA_ERR_ALIAS;
    // A window side wider than n + m reaches past every key: unbounded.
    const int64_t reach = (int64_t)n + m;
    const sdpa::MhaArgs a{x_q, x_kv, w_q, w_k, w_v, w_o, out, workspace, B, n, m, d_model, h, scale,
                          window_left > reach ? -1 : window_left,
                          window_right > reach ? -1 : window_right,
                          align == SDPA_ALIGN_BOTTOM_RIGHT ? 1 : 0, key_lens, d_k};
    clear_pending_error();
    const hipError_t e = sdpa::launch_mha_bf16(a, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

// ---- sdpa_forward_strided: q, k, v and out at any element strides.

namespace {

// One tensor's strides: batch, head and row stride (elements) for `len` rows
// of `width` elements.  Fills `s` and its byte span from the base pointer.
int check_strides(const int64_t* st, int32_t len, int32_t width, int32_t B, int32_t h, uint64_t esz,
                  sdpa::Strides* s, uint64_t* span) {
    const int64_t sb = st[0], sh = st[1], sr = st[2];
    const int64_t lim = (int64_t)1 << 40;
    if (sb < 0 || sh < 0 || sr < width || sb > lim || sh > lim || sr > lim) return SDPA_ERR_SHAPE;
    // every row starts 16-byte aligned
    if ((sb * (int64_t)esz) % 16 || (sh * (int64_t)esz) % 16 || (sr * (int64_t)esz) % 16)
        return SDPA_ERR_ALIGN;
    // 32-bit byte offsets within a head: its rows, and 64 rows from any tile start
    if ((uint64_t)((int64_t)(len - 1) * sr + width) * esz >= (1ull << 31)) return SDPA_ERR_SHAPE;
    if ((uint64_t)sr * esz * 64 >= (1ull << 31)) return SDPA_ERR_SHAPE;
    s->b = sb;
    s->h = sh;
    s->r = (int)sr;
    *span = (uint64_t)((int64_t)(B - 1) * sb + (int64_t)(h - 1) * sh + (int64_t)(len - 1) * sr + width) * esz;
    return SDPA_OK;
}

// The (batch, head, row) rows of the output, `width` elements each, are
// pairwise disjoint: taken in increasing stride order, every stride reaches
// past everything the smaller ones span.
bool rows_disjoint(const sdpa::Strides& s, int32_t B, int32_t h, int32_t n, int32_t width) {
    struct Dim { int64_t stride, extent; } d[3] = {{s.b, B}, {s.h, h}, {s.r, n}};
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (d[j].stride < d[i].stride) { const Dim t = d[i]; d[i] = d[j]; d[j] = t; }
    int64_t reach = width;  // elements spanned by one row
    for (const Dim& x : d) {
        if (x.extent == 1) continue;
        if (x.stride < reach) return false;
        reach += x.stride * (x.extent - 1);
    }
    return true;
}

}  // namespace

extern "C" int sdpa_forward_strided(const void* q, const void* k, const void* v, void* out, float* lse,
                                    int32_t B, int32_t h, int32_t n, int32_t m, int32_t d_k,
                                    int32_t d_v, float scale, int32_t window_left,
                                    int32_t window_right, int32_t align, const int32_t* key_lens,
                                    int32_t dtype, const int64_t* strides, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (!strides)
        return sdpa_forward_ex(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left,
                               window_right, align, key_lens, dtype, workspace, workspace_bytes,
                               stream);
    int st = validate_core(q, k, v, out, B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    int32_t wl, wr, br;
    st = window_args(n, m, window_left, window_right, align, &wl, &wr, &br);
    if (st != SDPA_OK) return st;
    const uint64_t esz = dtype == SDPA_F32 ? 4 : 2;
    sdpa::Layout lay{};
    uint64_t qs, ks, vs, os;
    if ((st = check_strides(strides + 0, n, d_k, B, h, esz, &lay.q, &qs)) != SDPA_OK) return st;
    if ((st = check_strides(strides + 3, m, d_k, B, h, esz, &lay.k, &ks)) != SDPA_OK) return st;
    if ((st = check_strides(strides + 6, m, d_v, B, h, esz, &lay.v, &vs)) != SDPA_OK) return st;
    if ((st = check_strides(strides + 9, n, d_v, B, h, esz, &lay.o, &os)) != SDPA_OK) return st;
    if (!rows_disjoint(lay.o, B, h, n, d_v)) return SDPA_ERR_ALIAS;
    const uint64_t heads = (uint64_t)B * h;
    struct Buf { const void* p; uint64_t n; };
    const Buf ins[] = {{q, qs}, {k, ks}, {v, vs}, {key_lens, key_lens ? (uint64_t)B * 4 : 0}};
    for (const Buf& b : ins)
        if (b.p && overlap(out, os, b.p, b.n)) return SDPA_ERR_ALIAS;
    if (lse) {
        if (reinterpret_cast<uintptr_t>(lse) & 3u) return SDPA_ERR_ALIGN;
        for (const Buf& b : ins)
            if (b.p && overlap(lse, heads * n * 4, b.p, b.n)) return SDPA_ERR_ALIAS;
        if (overlap(lse, heads * n * 4, out, os)) return SDPA_ERR_ALIAS;
    }
    const size_t need = forward_work_bytes(B, h, n, m, d_k, d_v, dtype);
    void* work = nullptr;
    if (workspace && need > 0) {
        if (!aligned16(workspace)) return SDPA_ERR_ALIGN;
        if (workspace_bytes < need) return SDPA_ERR_WORKSPACE;
        for (const Buf& b : ins)
            if (b.p && overlap(workspace, need, b.p, b.n)) return SDPA_ERR_ALIAS;
        if (overlap(workspace, need, out, os)) return SDPA_ERR_ALIAS;
        if (lse && overlap(workspace, need, lse, heads * n * 4)) return SDPA_ERR_ALIAS;
        work = workspace;
    }
    sdpa::Args a{q, k, v, out, B, h, n, m, scale, wl, wr, br, key_lens};
    a.lse = lse;
    a.d = d_k;
    a.dv = d_v;
    a.work = work;
    a.work_bytes = work ? workspace_bytes : 0;
    a.lay = lay;
    a.strided = true;
    return launch(a, dtype, stream);
}

// ---- sdpa_forward_ex_noalloc: the split-key workspace in static device memory.
//
// One array per GPU (each device that loads the library holds its own copy),
// reached through its device address, never through the host-side name.
static __device__ __align__(256) unsigned char scratch[SDPA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device; nullptr
// on a runtime error.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int sdpa_forward_ex_noalloc(const void* q, const void* k, const void* v, void* out,
                                       float* lse, int32_t B, int32_t h, int32_t n, int32_t m,
                                       int32_t d_k, int32_t d_v, float scale, int32_t window_left,
                                       int32_t window_right, int32_t align,
                                       const int32_t* key_lens, int32_t dtype, void* stream) {
    int st = validate(q, k, v, out, B, h, n, m, d_k, d_v, scale, key_lens, dtype);
    if (st != SDPA_OK) return st;
    int32_t wl, wr, br;
    st = window_args(n, m, window_left, window_right, align, &wl, &wr, &br);
    if (st != SDPA_OK) return st;
    if (lse) {
        if (reinterpret_cast<uintptr_t>(lse) & 3u) return SDPA_ERR_ALIGN;
        const uint64_t heads = (uint64_t)B * h, esz = dtype == SDPA_F32 ? 4 : 2;
        const struct { const void* p; uint64_t n; } ins[] = {
            {q, heads * n * d_k * esz}, {k, heads * m * d_k * esz}, {v, heads * m * d_v * esz},
            {out, heads * n * d_v * esz}, {key_lens, key_lens ? (uint64_t)B * 4 : 0}};
        for (const auto& b : ins)
            if (b.p && overlap(lse, heads * n * 4, b.p, b.n)) return SDPA_ERR_ALIAS;
    }
    const size_t need = forward_work_bytes(B, h, n, m, d_k, d_v, dtype);
    if (need > SDPA_NOALLOC_SCRATCH_BYTES) return SDPA_ERR_SCRATCH;
    sdpa::Args a{q, k, v, out, B, h, n, m, scale, wl, wr, br, key_lens};
    a.lse = lse;
    a.d = d_k;
    a.dv = d_v;
    if (need > 0) {
        void* work = scratch_on_current_device();
        if (!work) return SDPA_ERR_LAUNCH;
        a.work = work;
        a.work_bytes = SDPA_NOALLOC_SCRATCH_BYTES;
    }
    return launch(a, dtype, stream);
}

extern "C" const char* sdpa_strerror(int status) {
    switch (status) {
        case SDPA_OK: return "ok";
        case SDPA_ERR_NULL: return "a required pointer is NULL";
        case SDPA_ERR_SHAPE: return "bad shape: a dimension is < 1 or an element count overflows";
        case SDPA_ERR_UNSUPPORTED:
            return "unsupported: head widths are d_k = d_v = 64; bf16 attention also takes d_k = d_v = "
                   "16, 32, 128, 512 and d_v = 64 with d_k = 16 or 32; the backward pass takes d_k = d_v = "
                   "32, 64 or 128 in bf16 and 64 in fp32; the sublayer and dropout are bf16 with d_k = d_v "
                   "= 32, 64 or 128";
        case SDPA_ERR_ALIGN: return "a device pointer is not 16-byte aligned (key_lens: 4-byte)";
        case SDPA_ERR_MASK:
            return "bad mask: unknown mask_kind, causal with n != m, window side < -1 or unknown align";
        case SDPA_ERR_DTYPE: return "unknown dtype (SDPA_F32 = 0, SDPA_BF16 = 1)";
        case SDPA_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
        case SDPA_ERR_SCALE: return "scale (and keep_scale) must be finite and > 0";
        case SDPA_ERR_ALIAS: return "an output overlaps an input, the keep mask or another output";
        case SDPA_ERR_WORKSPACE: return "workspace smaller than its *_workspace_bytes size";
        case SDPA_ERR_SCRATCH:
            return "the call needs more split-key scratch than the library's static "
                   "SDPA_NOALLOC_SCRATCH_BYTES (use sdpa_forward_ex with a workspace)";
        default: return "unknown status";
    }
}

extern "C" int sdpa_version(void) { return kVersion; }
