// Fused single-pass attention forward for fp32 inputs on gfx950 (MI355X).
//
// Same computation as the bf16 kernel — Eq. (1) of 《精读 Attention Is All You
// Need：原始 Transformer 论文》, softmax(Q Kᵀ·scale) V per (batch, head), with
// illegal logits at −∞ (《Attention Is All You Need：注意力就是你所需要的一切》
// §3.2.3) — but fp32 end to end: fp32 products on the matrix cores
// (v_mfma_f32_32x32x2_f32), fp32 weights (no bf16 rounding anywhere), fp32
// output.  gfx950 has no reduced-precision fp32 (xf32) MFMA, so nothing is
// truncated.
//
// One wave owns 32 queries of one head; keys stream through LDS in tiles of 32
// rows.  Products are computed transposed (Sᵀ = K·Qᵀ, Oᵀ += Vᵀ·Pᵀ) so each lane
// holds one query's column, as in the bf16 kernel.  With one k value per lane
// per MFMA, Vᵀ is read straight from the row-major V tile (no transpose read).
//
// Accumulation across tiles is compensated (Kahan): each tile's Oᵀ part and
// weight sum are formed on top of what rounding has lost so far, then added
// into the running totals, and the new loss is kept for the next tile.  A plain running sum over L keys would round L/2 times in
// sequence, a first-order error of about L/2 · 2^-24 relative (0.25 at 2^23
// keys); compensated, the error stays at a few units of 2^-24 whatever L is.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int D = kHeadDim;  // 64
constexpr int BN = 32;       // keys per LDS tile
constexpr int QW = 32;       // queries per wave

// 16-byte chunk c (0..15) of tile row r sits at chunk position c ^ (r & 15).
__device__ __forceinline__ int swz16(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

template <int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_fwd_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, int BH, int H, int n, int m, float c_log2, int wl, int wr,
    int bottom_right, const int32_t* __restrict__ key_lens, int nqb, float* __restrict__ lse, Layout lay) {
    constexpr int NT = NW * 64;
    constexpr int CHUNKS = BN * D * 4 / 16;  // 512
    constexpr int CPT = (CHUNKS + NT - 1) / NT;

    __shared__ f32x4 sK[BN * 16];
    __shared__ f32x4 sV[BN * 16];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int g = blockIdx.x;
    const int bh = g % BH;
    const int qb = nqb - 1 - g / BH;
    const int b = bh / H;
    const int q0 = qb * (NW * QW);

    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    // Key tiles [tbeg, tend): the keys any query of the block may see (KeyWindow).
    const KeyWindow win{wl, wr, bottom_right ? L - n : 0, L};
    const int kbeg = win.lo(q0), kend = win.hi(min(q0 + NW * QW, n) - 1);
    const int tbeg = kbeg / BN;
    const int tend = kend > kbeg ? (kend + BN - 1) / BN : tbeg;

    const int hh = bh - b * H;
    const float* Qh = Q + head_offset(lay.q, b, hh);
    const float* Kh = K + head_offset(lay.k, b, hh);
    const float* Vh = V + head_offset(lay.v, b, hh);
    float* Oh = O + head_offset(lay.o, b, hh);

    // Qᵀ operand: MFMA step ks contracts d = ks (half-wave 0) and d = 32 + ks
    // (half-wave 1), so a lane keeps d = 32·hf + [0..31] of its query.
    const int qrow = q0 + w * QW + l32;
    float qop[32];
    if (qrow < n) {
        const f32x4* src = reinterpret_cast<const f32x4*>(Qh + (size_t)qrow * lay.q.r + 32 * hf);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const f32x4 x = src[c];
            qop[4 * c + 0] = x[0]; qop[4 * c + 1] = x[1]; qop[4 * c + 2] = x[2]; qop[4 * c + 3] = x[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) qop[i] = 0.f;
    }

    f32x4 rk[CPT], rv[CPT];
    auto gload = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            const int key = k0 + (c >> 4);
            if (c < CHUNKS && key < L) {
                rk[i] = reinterpret_cast<const f32x4*>(Kh + (size_t)key * lay.k.r)[c & 15];
                rv[i] = reinterpret_cast<const f32x4*>(Vh + (size_t)key * lay.v.r)[c & 15];
            } else {
                rk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                rv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto swrite = [&]() {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            if (c < CHUNKS) {
                const int idx = swz16(c >> 4, c & 15);
                sK[idx] = rk[i];
                sV[idx] = rv[i];
            }
        }
    };

    // Running Oᵀ and weight sum, and what rounding has lost from each so far
    // (to be added back).
    f32x16 oacc[2], ofix[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) { oacc[0][i] = oacc[1][i] = 0.f; ofix[0][i] = ofix[1][i] = 0.f; }
    float mrun = -INFINITY;
    float lrun = 0.f, lfix = 0.f;

    const int wq_lo = q0 + w * QW;
    const int wq_hi = min(wq_lo + QW, n) - 1;  // < wq_lo for a wave past n: empty
    const int my_q = wq_lo + l32;
    // Keys some query of the wave may see: [wlo, whi); legal for all: [flo, fhi).
    const bool wempty = wq_hi < wq_lo;
    const int wlo = wempty ? 0 : win.lo(wq_lo), whi = wempty ? 0 : win.hi(wq_hi);
    const int flo = wempty ? 0 : win.lo(wq_hi), fhi = wempty ? 0 : win.hi(wq_lo);
    const int qlo = win.lo(my_q), qhi = win.hi(my_q);
    const float* sVf = reinterpret_cast<const float*>(sV);

    if (tend > tbeg) gload(tbeg);
    for (int t = tbeg; t < tend; ++t) {
        __syncthreads();
        swrite();
        __syncthreads();
        if (t + 1 < tend) gload(t + 1);

        const int k0 = t * BN;
        if (k0 >= whi || k0 + BN <= wlo) continue;  // no query of this wave sees the tile

        // Sᵀ (32 keys × 32 queries) = K · Qᵀ, 32 steps of k = 2.
        f32x16 s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const f32x4 a4 = sK[swz16(l32, 8 * hf + c)];
#pragma unroll
            for (int e = 0; e < 4; ++e) s = mfma32x32x2_f32(a4[e], qop[4 * c + e], s);
        }

        const bool need_mask = k0 < flo || k0 + BN > fhi;
        if (need_mask) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + 8 * (i >> 2) + 4 * hf + (i & 3);
                if (key < qlo || key >= qhi) s[i] = -INFINITY;
            }
        }

        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[i]);
        mt = half_swap_max(mt);
        const float mnew = fmaxf(mrun, mt);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = exp2_hw((mrun - muse) * c_log2);
        mrun = mnew;
        const float mc = muse * c_log2;
        if (alpha != 1.f) {  // the running maximum moved: rescale totals and corrections
            lrun *= alpha;
            lfix *= alpha;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                oacc[0][i] *= alpha; oacc[1][i] *= alpha;
                ofix[0][i] *= alpha; ofix[1][i] *= alpha;
            }
        }
        float ly = lfix;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = exp2_hw(__builtin_fmaf(s[i], c_log2, -mc));
            s[i] = p;
            ly += p;
        }

        // This tile's Oᵀ part, Vᵀ · Pᵀ, accumulated onto the correction, so that
        // ofix becomes y = part + lost.  Step i contracts, for half-wave hf, the
        // key held in Sᵀ register i, i.e. tile row 8·(i/4) + 4·hf + i%4.
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 8 * (i >> 2) + 4 * hf + (i & 3);
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const int dv = 32 * dt + l32;
                const float a = sVf[swz16(r, dv >> 2) * 4 + (dv & 3)];
                ofix[dt] = mfma32x32x2_f32(a, s[i], ofix[dt]);
            }
        }
        // Kahan step: t = sum + y; lost = y − (t − sum); sum = t.
        {
#pragma clang fp contract(off)
            const float lt = lrun + ly;
            lfix = ly - (lt - lrun);
            lrun = lt;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float y = ofix[dt][i];
                    const float t = oacc[dt][i] + y;
                    ofix[dt][i] = y - (t - oacc[dt][i]);
                    oacc[dt][i] = t;
                }
        }
    }

#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] += ofix[dt][i];
    const float ltot = half_swap_sum(lrun + lfix);
    if (qrow < n) {
        float* dst = Oh + (size_t)qrow * lay.o.r;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int dv = 32 * dt + 8 * i4 + 4 * hf;
                f32x4 o;
                // True division (within an ulp).  ltot = 0 (no legal key) gives a
                // zero row; a NaN ltot (NaN among the legal inputs) stays NaN.
                o[0] = ltot != 0.f ? oacc[dt][4 * i4 + 0] / ltot : 0.f;
                o[1] = ltot != 0.f ? oacc[dt][4 * i4 + 1] / ltot : 0.f;
                o[2] = ltot != 0.f ? oacc[dt][4 * i4 + 2] / ltot : 0.f;
                o[3] = ltot != 0.f ? oacc[dt][4 * i4 + 3] / ltot : 0.f;
                *reinterpret_cast<f32x4*>(dst + dv) = o;
            }
        // Natural-log log-sum-exp of the scaled logits, relative to the final
        // running maximum (−∞ for a query with no legal key: ltot = 0).
        if (lse && hf == 0) {
            const float mc = (mrun == -INFINITY ? 0.f : mrun) * c_log2;
            lse[(size_t)bh * n + qrow] = (mc + log2f(ltot)) * 0.6931471805599453f;
        }
    }
}

}  // namespace

hipError_t launch_f32_long(const Args& a, hipStream_t stream) {
    // Two waves per workgroup at every n: for n <= 32 the second wave has no
    // queries and only shares the tile loads (its tile loop skips the math),
    // which keeps each lane's staging registers at four 16-byte chunks.
    constexpr int NW = 2;
    const int BH = a.B * a.H;
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);
    const int nqb = (a.n + NW * QW - 1) / (NW * QW);
    hipLaunchKernelGGL(sdpa_fwd_f32<NW>, dim3(nqb * BH), dim3(NW * 64), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.out,
                       BH, a.H, a.n, a.m, c_log2, a.wl, a.wr, a.bottom_right, a.key_lens, nqb, a.lse, a.lay);
    return hipGetLastError();
}

hipError_t launch_f32(const Args& a0, hipStream_t stream) {
    Args a = a0;
    if (!a.strided) a.lay = dense_layout(a.H, a.n, a.m, a.d, a.d);  // packed layout
    return short_f32_fits(a) ? launch_f32_short(a, stream) : launch_f32_long(a, stream);
}

}  // namespace sdpa
