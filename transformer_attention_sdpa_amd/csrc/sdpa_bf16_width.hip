// Eq. (1) in bf16 for head widths other than the 64-wide kernels' one:
// d_k, d_v ∈ {16, 32, 64, 128} in the combinations listed by width_supported.
//
// The pages' model variants change the head widths (《精读 Attention Is All
// You Need：原始 Transformer 论文》 Table 3: row (A) runs h = 4, 16 and 32 heads of
// 128, 32 and 16 next to the base model's 8 heads of 64; row (B) shrinks the
// key width d_k to 16 or 32 and keeps d_v = 64; row (C) pairs d_model = 256
// with 32-wide heads and d_model = 1024 with 128-wide ones).  The 64-wide
// kernels are tuned to their one width; this one is written once for any
// pair of widths, with the same transposed products:
//
//   Sᵀ (64 keys × 32 queries)  = K · Qᵀ      A = K rows from LDS, B = Qᵀ in VGPRs
//   Oᵀ (d_v × 32 queries)     += Vᵀ · Pᵀ    A = Vᵀ via LDS transpose reads,
//                                           B = Pᵀ from the Sᵀ registers
//
// on v_mfma_f32_32x32x16_bf16 (its 16-long contraction is one k-step at
// d_k = 16; at d_v = 16 the upper half of the 32-row Oᵀ block is computed
// and dropped), one 32-query block per wave, 64-key tiles double-buffered in
// LDS by buffer_load … lds, and an exact online softmax (the tile maximum
// moves the reference every tile).  Key windows, key lengths, the
// log-sum-exp output and attention dropout (at d_k = d_v = 32 and 128) behave
// exactly as in the 64-wide kernels.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int BT = 64;  // keys per LDS tile

// 16-byte chunk position of chunk c of row r in a tile with D/8 chunks per
// row, XOR-swizzled so that 16 consecutive rows read at one chunk (one
// 16-byte MFMA operand per lane) fall on distinct banks of gfx950's 256-byte
// LDS pass: 32-byte rows (D = 16) share a pass eight at a time, 64-byte rows
// (D = 32) four at a time, 256-byte rows (D = 128) fill it alone.  The
// transpose reads of Vᵀ take rows 4·G' + [0..3] at four consecutive chunks of
// one 4-chunk group; at D = 128 the row's low two bits therefore pick the
// chunk group (bits 2–3 of the XOR) and its next two bits the chunk within
// it, which spreads those reads over all banks as well (an XOR with r mod 16
// alone keeps them inside one group: four-way conflicts).
template <int D>
__device__ __forceinline__ int wswz(int r, int c) {
    if constexpr (D == 16) return r * 2 + (c ^ ((r >> 3) & 1));
    else if constexpr (D == 32) return r * 4 + (c ^ ((r >> 2) & 3));
    else if constexpr (D == 128) return r * 16 + (c ^ (((r & 3) << 2) | ((r >> 2) & 3)));
    else return lds_swz(r, c);
}

__device__ __forceinline__ u32x4 wds_read_b128(uint32_t a) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
__device__ __forceinline__ u32x2 wds_read_tr(uint32_t a) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
template <int N>
__device__ __forceinline__ void wlds_wait(u32x4 (&x)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}
template <int N>
__device__ __forceinline__ void wlds_wait(u32x2 (&x)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}

// STRIDED: runtime strides of `lay`; else the packed layout, compile-time.
// DROP: attention dropout with keep-bit words [BH, n, ⌈m/32⌉]: the dropped
// weights leave the P·V product but not the row sums, and the output is
// scaled by keep_scale.
template <int DK, int DV, int NW, bool STRIDED, bool DROP>
__global__ __launch_bounds__(NW * 64) void sdpa_fwd_bf16_width(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ lse, int BH, int H, int n, int m, float c_log2, int wl,
    int wr, int bottom_right, const int32_t* __restrict__ key_lens, int nqb, Layout lay,
    const uint32_t* __restrict__ keep, float keep_scale) {
    constexpr int KS = DK / 16;               // k-steps of the score product
    constexpr int DT = (DV + 31) / 32;        // 32-row blocks of Oᵀ
    constexpr int CPK = DK / 8, CPV = DV / 8; // 16-byte chunks per K / V row
    constexpr int TK = BT * DK * 2, TV = BT * DV * 2;  // bytes per K / V tile
    constexpr int NLK = TK / 1024, NLV = TV / 1024;    // 1 KiB loads per tile
    constexpr int LPK = (NLK + NW - 1) / NW, LPV = (NLV + NW - 1) / NW;  // per wave, at most
    static_assert(DK % 16 == 0 && DV % 16 == 0 && NLK >= 1 && NLV >= 1, "width");
    static_assert(NW * 32 * DV * 2 <= 2 * (TK + TV), "output staging");
    __shared__ __attribute__((aligned(1024))) char lds[2 * (TK + TV)];  // [buf][K | V]

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5, gi = lane & 15;

    // Latest query blocks first (they see the most keys under a causal mask).
    const int g = blockIdx.x;
    const int bh = g % BH;
    const int q0 = (nqb - 1 - g / BH) * 32 * NW;
    const int b = bh / H;
    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    const KeyWindow win{wl, wr, bottom_right ? L - n : 0, L};
    const int qlast = min(q0 + 32 * NW, n) - 1;
    const int kbeg = win.lo(q0), kend = win.hi(qlast);
    const int tbeg = kbeg / BT;
    const int tend = kend > kbeg ? (kend + BT - 1) / BT : tbeg;
    const int wq0 = q0 + 32 * w;
    const int wlast = min(wq0 + 32, n) - 1;
    const bool wact = wlast >= wq0;
    const int wlo = wact ? win.lo(wq0) : 0, whi = wact ? win.hi(wlast) : 0;
    const int flo = wact ? win.lo(wlast) : 0, fhi = wact ? win.hi(wq0) : 0;

    const int hh = bh - b * H;
    const uint16_t* Qh = Q + (STRIDED ? head_offset(lay.q, b, hh) : (long long)bh * n * DK);
    const uint16_t* Kh = K + (STRIDED ? head_offset(lay.k, b, hh) : (long long)bh * m * DK);
    const uint16_t* Vh = V + (STRIDED ? head_offset(lay.v, b, hh) : (long long)bh * m * DV);
    uint16_t* Oh = O + (STRIDED ? head_offset(lay.o, b, hh) : (long long)bh * n * DV);
    const int qr = STRIDED ? lay.q.r : DK, kr = STRIDED ? lay.k.r : DK;
    const int vr = STRIDED ? lay.v.r : DV, orr = STRIDED ? lay.o.r : DV;
    const int qrow = wq0 + l32;
    const bool qok = qrow < n;
    // Dropout: this lane's row of keep words (rows past n read row n − 1;
    // their outputs are not stored).
    const int kwords = (m + 31) >> 5;
    const uint32_t* krow = DROP ? keep + ((size_t)bh * n + min(qrow, n - 1)) * kwords : nullptr;
    // Qᵀ as the B operand: dims 16·ks + 8·hf + [0..7] of this lane's query.
    bf16x8 qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qop[ks] = qok ? __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * qr)[2 * ks + hf])
                      : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});

    // Per-lane LDS offsets: the K operand of k-step ks (row l32, chunk 2·ks + hf)
    // and the Vᵀ transpose reads (rows 4·hf + gi/4, + 8; k-step j adds 16·j rows,
    // which leaves the swizzle of these rows unchanged for every width here).
    // At d_v = 16 the lanes of dims 16..31 read dims 0..15 again: those rows of
    // Oᵀ are never stored.
    int kaddr[KS], vaddr[DT][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kaddr[ks] = wswz<DK>(l32, 2 * ks + hf) * 16;
    {
        const int r0 = 4 * hf + (gi >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int c0 = (32 * dt + 16 * ((lane >> 4) & 1) + 4 * (gi & 3)) & (DV >= 32 ? 1023 : DV - 1);
            vaddr[dt][0] = wswz<DV>(r0, c0 >> 3) * 16 + (c0 & 7) * 2;
            vaddr[dt][1] = wswz<DV>(r0 + 8, c0 >> 3) * 16 + (c0 & 7) * 2;
        }
    }
    // Tile loads: 1 KiB load u of a tile fills rows (1024 / row bytes)·u + lane/CP;
    // wave w issues loads w, w + NW, … of each tensor.
    int ldk_off[LPK], ldk_lds[LPK], ldv_off[LPV], ldv_lds[LPV];
#pragma unroll
    for (int u = 0; u < LPK; ++u) {
        const int blk = w + NW * u;
        const int row = (1024 / (DK * 2)) * blk + lane / CPK, pos = lane % CPK;
        // the chunk whose swizzled position is pos (XOR is its own inverse)
        ldk_off[u] = row * kr * 2 + (wswz<DK>(row, pos) - row * CPK) * 16;
        ldk_lds[u] = blk * 1024;
    }
#pragma unroll
    for (int u = 0; u < LPV; ++u) {
        const int blk = w + NW * u;
        const int row = (1024 / (DV * 2)) * blk + lane / CPV, pos = lane % CPV;
        ldv_off[u] = row * vr * 2 + (wswz<DV>(row, pos) - row * CPV) * 16;
        ldv_lds[u] = TK + blk * 1024;
    }
    auto issue = [&](int t, int buf) {
        // buffer ranges end with the last legal row
        const i32x4 rk = make_rsrc(Kh + (size_t)t * BT * kr, rows_span(L - t * BT, kr, DK, 2));
        const i32x4 rv = make_rsrc(Vh + (size_t)t * BT * vr, rows_span(L - t * BT, vr, DV, 2));
        char* base = lds + buf * (TK + TV);
#pragma unroll
        for (int u = 0; u < LPK; ++u)
            if (NLK % NW == 0 || w + NW * u < NLK) load16_to_lds(rk, base + ldk_lds[u], ldk_off[u]);
#pragma unroll
        for (int u = 0; u < LPV; ++u)
            if (NLV % NW == 0 || w + NW * u < NLV) load16_to_lds(rv, base + ldv_lds[u], ldv_off[u]);
    };

    const uint32_t l0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    float mref = -INFINITY, lsum = 0.f;

    if (tend > tbeg) issue(tbeg, 0);
    wait_vmem();
    __syncthreads();
    for (int t = tbeg; t < tend; ++t) {
        const int buf = (t - tbeg) & 1;
        if (t + 1 < tend) issue(t + 1, buf ^ 1);
        const int k0 = t * BT;
        if (k0 < whi && k0 + BT > wlo) {  // uniform: some query of the wave sees the tile
            const uint32_t sk = l0 + buf * (TK + TV), sv = sk + TK;
            uint32_t kw[2] = {0u, 0u};  // keep words of keys k0..k0+31 and k0+32..k0+63
            if constexpr (DROP) {
                const int w0 = k0 >> 5;
                kw[0] = w0 < kwords ? krow[w0] : 0u;
                kw[1] = w0 + 1 < kwords ? krow[w0 + 1] : 0u;
            }
            f32x16 s[2];
            {
                u32x4 a[2 * KS];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) a[kt * KS + ks] = wds_read_b128(sk + kaddr[ks] + kt * 32 * DK * 2);
                wlds_wait(a);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        s[kt] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, a[kt * KS + ks]), qop[ks], s[kt]);
                }
            }
            // Register i of s[kt] is key k0 + 32·kt + 8·(i/4) + 4·hf + i%4.
            if (k0 < flo || k0 + BT > fhi) {
                const int llo = win.lo(qrow) - k0 - 4 * hf, lhi = win.hi(qrow) - k0 - 4 * hf;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int off = 32 * kt + 8 * (i >> 2) + (i & 3);
                        s[kt][i] = (off >= llo && off < lhi) ? s[kt][i] : -INFINITY;
                    }
            }
            // Exact online softmax: move the reference to the running maximum.
            float x = s[0][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) x = fmaxf(x, s[0][i]);
#pragma unroll
            for (int i = 0; i < 16; ++i) x = fmaxf(x, s[1][i]);
            const float mnew = fmaxf(mref, half_swap_max(x));
            // mref = −∞: nothing accumulated yet (alpha multiplies zeros);
            // mnew = −∞: no legal key so far, keep alpha = 1.
            const float alpha = mnew == -INFINITY ? 1.f : exp2_hw((mref - mnew) * c_log2);
            mref = mnew;
            const float mc = (mnew == -INFINITY ? 0.f : mnew) * c_log2;
            lsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
            bf16x8 pb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kt = j >> 1, vb = 8 * (j & 1);
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = exp2_hw(__builtin_fmaf(s[kt][vb + e], c_log2, -mc));
                    lsum += p[e];
                }
                pb[j] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
                // Dropout, after the row sum has counted the weights: element e
                // of pb[j] is key 16·(j%2) + 4·hf + e (e < 4) or + 8 + (e − 4) of
                // word kt.
                if constexpr (DROP) {
                    const uint32_t wd = kw[kt] >> (16 * (j & 1) + 4 * hf);
                    pb[j] = keep_pairs(pb[j], wd);
                }
            }
            // Oᵀ += Vᵀ · Pᵀ.
            u32x2 va[4 * DT * 2];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    va[(j * DT + dt) * 2] = wds_read_tr(sv + vaddr[dt][0] + j * 16 * DV * 2);
                    va[(j * DT + dt) * 2 + 1] = wds_read_tr(sv + vaddr[dt][1] + j * 16 * DV * 2);
                }
            wlds_wait(va);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x2 lo = va[(j * DT + dt) * 2], hi = va[(j * DT + dt) * 2 + 1];
                    const u32x4 v4 = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[dt] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, v4), pb[j], oacc[dt]);
                }
        }
        wait_vmem();
        __syncthreads();
    }

    // Oᵀ / l and store: register i of oacc[dt] is dim 32·dt + 8·(i/4) + 4·hf + i%4.
    const float ltot = half_swap_sum(lsum);
    // no legal key ⇒ zero row; a NaN sum (NaN legal inputs) stays NaN
    const float inv = ltot != 0.f ? (DROP ? keep_scale : 1.f) / ltot : 0.f;
    if (qok && lse && hf == 0) {
        const float mc = (mref == -INFINITY ? 0.f : mref) * c_log2;
        lse[(size_t)bh * n + qrow] = (mc + log2f(ltot)) * 0.6931471805599453f;
    }
    // The output rows go through a wave-private LDS area (the tiles are free:
    // every wave passed the loop's last barrier after its last read), so that
    // the stores write 16 bytes a lane along rows.  Register i of oacc[dt] is
    // dim 32·dt + 8·(i/4) + 4·hf + i%4 of row l32; 16-byte chunk c of a row
    // sits at position c ^ (row mod CPV).
    char* area = lds + w * 32 * DV * 2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int col = 32 * dt + 8 * i4 + 4 * hf;
            if (DV >= 32 || 8 * i4 < DV) {  // at d_v = 16, dims 16..31 are the dropped half
                bf16x4 o;
                o[0] = (__bf16)(oacc[dt][4 * i4 + 0] * inv);
                o[1] = (__bf16)(oacc[dt][4 * i4 + 1] * inv);
                o[2] = (__bf16)(oacc[dt][4 * i4 + 2] * inv);
                o[3] = (__bf16)(oacc[dt][4 * i4 + 3] * inv);
                const int pos = (col >> 3) ^ (l32 & (CPV - 1));
                *reinterpret_cast<bf16x4*>(area + (l32 * CPV + pos) * 16 + (col & 7) * 2) = o;
            }
        }
#pragma unroll
    for (int k = 0; k < CPV / 2; ++k) {
        const int id = lane + 64 * k;
        const int row = id / CPV, c = id % CPV;
        const u32x4 x = *reinterpret_cast<const u32x4*>(area + (row * CPV + (c ^ (row & (CPV - 1)))) * 16);
        if (wq0 + row < n) store16_nt(Oh + (size_t)(wq0 + row) * orr + 8 * c, x);
    }
}

template <int DK, int DV, int NW>
hipError_t launch_width_nw(const Args& a, hipStream_t stream) {
    const int BH = a.B * a.H;
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    const int nqb = (a.n + 32 * NW - 1) / (32 * NW);
    const auto kernel = a.keep ? (a.strided ? sdpa_fwd_bf16_width<DK, DV, NW, true, true>
                                            : sdpa_fwd_bf16_width<DK, DV, NW, false, true>)
                               : (a.strided ? sdpa_fwd_bf16_width<DK, DV, NW, true, false>
                                            : sdpa_fwd_bf16_width<DK, DV, NW, false, false>);
    hipLaunchKernelGGL(kernel, dim3(nqb * BH), dim3(NW * 64), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.out,
                       a.lse, BH, a.H, a.n, a.m, c_log2, a.wl, a.wr, a.bottom_right, a.key_lens, nqb, a.lay,
                       a.keep, a.keep_scale);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_width(const Args& a, hipStream_t stream) {
    // 4 waves (128 queries) per workgroup once there are enough blocks.
    if ((long long)a.B * a.H * ((a.n + 127) / 128) >= 1024) return launch_width_nw<DK, DV, 4>(a, stream);
    return launch_width_nw<DK, DV, 2>(a, stream);
}

}  // namespace

bool width_supported(int d_k, int d_v) {
    if (d_k == d_v) return d_k == 16 || d_k == 32 || d_k == 64 || d_k == 128 || d_k == 512;
    return d_v == 64 && (d_k == 16 || d_k == 32);
}

hipError_t launch_bf16_width(const Args& a, hipStream_t stream) {
    if (a.d == 16 && a.dv == 16) return launch_width<16, 16>(a, stream);
    if (a.d == 32 && a.dv == 32) return launch_width<32, 32>(a, stream);
    if (a.d == 128 && a.dv == 128) return launch_width<128, 128>(a, stream);
    if (a.d == 16 && a.dv == 64) return launch_width<16, 64>(a, stream);
    if (a.d == 32 && a.dv == 64) return launch_width<32, 64>(a, stream);
    if (a.d == 512 && a.dv == 512) return launch_bf16_wide(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
