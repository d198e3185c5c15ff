// Eq. (1) in bf16 at d_k = d_v = 512: one head as wide as the model
// (《精读 Attention Is All You Need：原始 Transformer 论文》 Table 3, row (A):
// h = 1 with d_k = d_v = 512 beside the base model's 8 heads of 64).
//
// At this width a query's operands no longer fit in registers (512 dims are
// 64 VGPRs per sub-block of 32 queries), so a workgroup keeps its 32 queries
// in LDS and splits the head dimension over its four waves:
//
//   partial Sᵀ_w (32 keys × 32 queries) = K_w · Q_wᵀ over dims [128w, 128w + 128)
//   Sᵀ = Σ_w partial Sᵀ_w   (through LDS, summed in wave order by every wave)
//   Oᵀ_w (128 dims × 32 queries) += V_wᵀ · Pᵀ over output dims [128w, 128w + 128)
//
// on v_mfma_f32_32x32x16_bf16, with 32-key tiles of K and V (32 KiB each) and
// an exact online softmax (the tile maximum moves the reference every tile),
// computed identically by every wave from the same summed scores.  Rows of
// 1 KiB are swizzled by 16-byte chunk (chunk c of row r at c ^ g(r), g(r) =
// 4·(r mod 4) + (r / 4) mod 4), so the 16 rows that one operand read touches
// fall on distinct banks, and so do the transpose reads of Vᵀ, whose rows
// 4·G' + [0..3] take four consecutive chunks of one 4-chunk group (g's low
// bits alone would keep them in one group of 16 banks); one 1 KiB
// buffer_load … lds fills one row.  Key windows, key lengths, the
// log-sum-exp output and caller strides behave as in the other kernels.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int WD = 512;           // head width
constexpr int WCH = WD / 8;       // 16-byte chunks per row
constexpr int ROWB = WD * 2;      // bytes per row
constexpr int WBT = 32;           // keys per tile
constexpr int WBQ = 32;           // queries per workgroup
constexpr int WNW = 4;            // waves
constexpr int WSLICE = WD / WNW;  // dims per wave (128)
constexpr int LQ = 0, LK = WBQ * ROWB, LV = LK + WBT * ROWB, LRED = LV + WBT * ROWB;
constexpr int LDS_BYTES = LRED + WNW * 4096;  // Q, K, V (32 KiB each), partial scores (16 KiB)

// The chunk swizzle g(r) of row r, and the byte offset of 16-byte chunk c of row r.
__device__ __forceinline__ int wide_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int wide_off(int r, int c) { return (r * WCH + (c ^ wide_swz(r))) * 16; }

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

// Rows [8w, 8w + 8) of a 32-row block from `base` (row stride `rs` elements,
// `rows` legal rows from base on) into LDS at `dst`: one 1 KiB load per row,
// lane p bringing the chunk whose swizzled position is p.
__device__ __forceinline__ void load_rows(char* dst, const uint16_t* base, int rs, int rows, int w, int lane) {
    const i32x4 rsrc = make_rsrc(base, rows_span(rows, rs, WD, 2));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 8 * w + i;
        load16_to_lds(rsrc, dst + r * ROWB, r * rs * 2 + ((lane ^ wide_swz(r)) * 16));
    }
}

// NS: the workgroups that share one query block, each producing WD / NS of
// the output dims (every one forms the whole scores; 2 when the query blocks
// alone would leave compute units idle).
template <int NS>
__global__ __launch_bounds__(WNW * 64) void sdpa_fwd_bf16_wide(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ lse, int BH, int H, int n, int m, float c_log2, int wl,
    int wr, int bottom_right, const int32_t* __restrict__ key_lens, int nqb, Layout lay) {
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5, gi = lane & 15;

    constexpr int OSLICE = WD / NS / WNW;  // output dims per wave
    const int sidx = NS == 1 ? 0 : (int)(blockIdx.x % NS);  // this workgroup's share of the output dims
    const int g = blockIdx.x / NS;
    const int bh = g % BH;
    const int q0 = (nqb - 1 - g / BH) * WBQ;  // latest query blocks first
    const int b = bh / H, hh = bh - b * H;
    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    const KeyWindow win{wl, wr, bottom_right ? L - n : 0, L};
    const int qlast = min(q0 + WBQ, n) - 1;
    const int kbeg = win.lo(q0), kend = win.hi(qlast);
    const int tb = kbeg / WBT;
    const int te = kend > kbeg ? (kend + WBT - 1) / WBT : tb;
    const int flo = win.lo(qlast), fhi = win.hi(q0);  // legal for every query of the block

    const uint16_t* Qh = Q + head_offset(lay.q, b, hh);
    const uint16_t* Kh = K + head_offset(lay.k, b, hh);
    const uint16_t* Vh = V + head_offset(lay.v, b, hh);
    uint16_t* Oh = O + head_offset(lay.o, b, hh);
    const int qrow = q0 + l32;

    // Per-lane LDS offsets: score operands of k-step ks (row l32, chunk 2·ks + hf)
    // and the Vᵀ transpose reads of this wave's output dims (rows 4·hf + gi/4,
    // + 8; k-step j adds 16·j rows, which keeps the swizzle).
    const uint32_t l0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
    int vaddr[OSLICE / 32][2];
    {
        const int r0 = 4 * hf + (gi >> 2);
#pragma unroll
        for (int dt = 0; dt < OSLICE / 32; ++dt) {
            const int c0 = (WD / NS) * sidx + OSLICE * w + 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
            vaddr[dt][0] = LV + wide_off(r0, c0 >> 3) + (c0 & 7) * 2;
            vaddr[dt][1] = LV + wide_off(r0 + 8, c0 >> 3) + (c0 & 7) * 2;
        }
    }

    f32x16 oacc[OSLICE / 32];
#pragma unroll
    for (int dt = 0; dt < OSLICE / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
    float mref = -INFINITY, lsum = 0.f;

    if (te > tb) {
        load_rows(lds + LQ, Qh + (size_t)q0 * lay.q.r, lay.q.r, n - q0, w, lane);
        load_rows(lds + LK, Kh + (size_t)tb * WBT * lay.k.r, lay.k.r, L - tb * WBT, w, lane);
        load_rows(lds + LV, Vh + (size_t)tb * WBT * lay.v.r, lay.v.r, L - tb * WBT, w, lane);
    }
    for (int t = tb; t < te; ++t) {
        const int k0 = t * WBT;
        wait_vmem();
        __syncthreads();  // K and V of tile t (and Q) are in LDS
        // Partial Sᵀ over this wave's dims; register i is key k0 + 8·(i/4) + 4·hf + i%4.
        f32x16 sp;
#pragma unroll
        for (int i = 0; i < 16; ++i) sp[i] = 0.f;
        {
            u32x4 a[16];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int c = 2 * (8 * w + ks) + hf;
                a[2 * ks] = wds_read_b128(l0 + LK + wide_off(l32, c));
                a[2 * ks + 1] = wds_read_b128(l0 + LQ + wide_off(l32, c));
            }
            wlds_wait(a);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                sp = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, a[2 * ks]), __builtin_bit_cast(bf16x8, a[2 * ks + 1]),
                                       sp);
        }
        {
            // [wave][q4][lane]: consecutive lanes write consecutive 16 bytes
            u32x4* red = reinterpret_cast<u32x4*>(lds + LRED + w * 4096 + lane * 16);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) red[64 * q4] = u32x4{__float_as_uint(sp[4 * q4]), __float_as_uint(sp[4 * q4 + 1]),
                                                           __float_as_uint(sp[4 * q4 + 2]),
                                                           __float_as_uint(sp[4 * q4 + 3])};
        }
        __syncthreads();  // every partial written; every read of K(t) done
        if (t + 1 < te)
            load_rows(lds + LK, Kh + (size_t)(t + 1) * WBT * lay.k.r, lay.k.r, L - (t + 1) * WBT, w, lane);
        // Sᵀ = Σ partials in wave order (the same sum in every wave).
        f32x16 s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < WNW; ++w2) {
            const u32x4* red = reinterpret_cast<const u32x4*>(lds + LRED + w2 * 4096 + lane * 16);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const u32x4 x = red[64 * q4];
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * q4 + e] += __uint_as_float(x[e]);
            }
        }
        if (k0 < flo || k0 + WBT > fhi) {  // −∞ on illegal logits
            const int llo = win.lo(qrow) - k0 - 4 * hf, lhi = win.hi(qrow) - k0 - 4 * hf;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 8 * (i >> 2) + (i & 3);
                s[i] = (off >= llo && off < lhi) ? s[i] : -INFINITY;
            }
        }
        // Exact online softmax.
        float x = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) x = fmaxf(x, s[i]);
        const float mnew = fmaxf(mref, half_swap_max(x));
        const float alpha = mnew == -INFINITY ? 1.f : exp2_hw((mref - mnew) * c_log2);
        mref = mnew;
        const float mc = (mnew == -INFINITY ? 0.f : mnew) * c_log2;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < OSLICE / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
        bf16x8 pb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = exp2_hw(__builtin_fmaf(s[8 * j + e], c_log2, -mc));
                lsum += p[e];
            }
            pb[j] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        }
        // Oᵀ_w += V_wᵀ · Pᵀ.
        {
            u32x2 va[2 * (OSLICE / 32) * 2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int dt = 0; dt < OSLICE / 32; ++dt) {
                    va[(j * (OSLICE / 32) + dt) * 2] = wds_read_tr(l0 + vaddr[dt][0] + j * 16 * ROWB);
                    va[(j * (OSLICE / 32) + dt) * 2 + 1] = wds_read_tr(l0 + vaddr[dt][1] + j * 16 * ROWB);
                }
            wlds_wait(va);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int dt = 0; dt < OSLICE / 32; ++dt) {
                    const u32x2 lo = va[(j * (OSLICE / 32) + dt) * 2], hi = va[(j * (OSLICE / 32) + dt) * 2 + 1];
                    const u32x4 v4 = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[dt] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, v4), pb[j], oacc[dt]);
                }
        }
        __syncthreads();  // every read of V(t) and of the partials done
        if (t + 1 < te)
            load_rows(lds + LV, Vh + (size_t)(t + 1) * WBT * lay.v.r, lay.v.r, L - (t + 1) * WBT, w, lane);
    }

    wait_vmem();  // (no copy into LDS outlives the loop)

    // Oᵀ / l: register i of oacc[dt] is dim 128·w + 32·dt + 8·(i/4) + 4·hf + i%4 of query q0 + l32.
    const float ltot = half_swap_sum(lsum);
    const float inv = ltot != 0.f ? 1.f / ltot : 0.f;  // no legal key ⇒ zero row
    if (qrow < n) {
        if (lse && sidx == 0 && w == 0 && hf == 0) {
            const float mc = (mref == -INFINITY ? 0.f : mref) * c_log2;
            lse[(size_t)bh * n + qrow] = (mc + log2f(ltot)) * 0.6931471805599453f;
        }
        uint16_t* dst = Oh + (size_t)qrow * lay.o.r + (WD / NS) * sidx + OSLICE * w;
#pragma unroll
        for (int dt = 0; dt < OSLICE / 32; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                bf16x4 o;
                o[0] = (__bf16)(oacc[dt][4 * i4 + 0] * inv);
                o[1] = (__bf16)(oacc[dt][4 * i4 + 1] * inv);
                o[2] = (__bf16)(oacc[dt][4 * i4 + 2] * inv);
                o[3] = (__bf16)(oacc[dt][4 * i4 + 3] * inv);
                *reinterpret_cast<bf16x4*>(dst + 32 * dt + 8 * i4 + 4 * hf) = o;
            }
    }
}

}  // namespace

hipError_t launch_bf16_wide(const Args& a, hipStream_t stream) {
    const int BH = a.B * a.H;
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    const int nqb = (a.n + WBQ - 1) / WBQ;
    // Two workgroups per query block (each half of the output dims) while the
    // query blocks alone are fewer than the compute units.
    const bool split = (long long)nqb * BH < 256;
    const auto kernel = split ? sdpa_fwd_bf16_wide<2> : sdpa_fwd_bf16_wide<1>;
    hipLaunchKernelGGL(kernel, dim3(nqb * BH * (split ? 2 : 1)), dim3(WNW * 64), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.out, a.lse, BH, a.H, a.n, a.m,
                       c_log2, a.wl, a.wr, a.bottom_right, a.key_lens, nqb, a.lay);
    return hipGetLastError();
}

}  // namespace sdpa
