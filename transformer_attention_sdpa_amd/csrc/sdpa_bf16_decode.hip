// Decoder-step attention forward (n <= 16 queries per head, m > 64 keys), bf16,
// gfx950.
//
// One autoregressive step of the decoder (《Attention Is All You Need：注意力
// 就是你所需要的一切》 §3.1: the decoder consumes the symbols it generated
// before) asks a few new queries per sequence against all of that sequence's
// cached keys.  The work per key is a 64-wide dot product for each of ≤ 16
// queries, so the step is bound by reading K and V from HBM, and the kernel is
// built to keep many K/V bytes in flight:
//
//   * one workgroup of four waves per (batch, head); the key range any query
//     may see (KeyWindow, usually bottom-right causal) is cut into 32-key steps
//     and the waves take contiguous runs of steps, each with its own online
//     softmax, so no workgroup barrier sits in the loop;
//   * K goes straight from HBM into VGPRs as the A operand of
//     v_mfma_f32_16x16x32_bf16 (Sᵀ = K·Qᵀ, the same transposed form as the other
//     kernels: each lane owns one query column); V goes HBM → LDS with
//     buffer_load … lds into the wave's own double-buffered slice and is read
//     back transposed (ds_read_b64_tr_b16) for Oᵀ += Vᵀ·Pᵀ;
//   * the next step's K and V are requested before the current step's math;
//   * buffer ranges end at the key length, so rows past it are never read;
//   * at the end the four waves' (max, sum, Oᵀ) are merged through LDS with the
//     usual rescale by exp(max_w − max) and the output is normalised once.
//
// Arithmetic contract as in the other bf16 kernels: fp32 scores and softmax,
// −∞ on illegal logits, weights rounded to bf16 for P·V with fp32
// accumulation, output rounded once to bf16.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int D = kHeadDim;  // 64
constexpr int QN = 16;       // query columns per head (n <= QN)
constexpr int NWD = 4;       // waves per workgroup
constexpr int PREC = 4 + 64; // floats per (split, head, query) record of the split mode

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float quad_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return half_swap_max(max2(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return half_swap_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}
extern "C" __device__ i32x4 sdpa_dec_buffer_load_v4i32(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

// KS keys per step (a multiple of 32): NTL tiles of 16 keys for the scores, NJ
// k-steps of 32 keys for P·V, NVL loads of 1 KiB (8 V rows) per step.
// HPW heads per workgroup, NWD / HPW waves each: several short caches share a
// workgroup, so that all heads fit on the GPU in one round of workgroups.
// STRIDED: runtime strides of `lay` (else the packed layout, compile-time).
template <int KS, int HPW, bool STRIDED>
__global__ __launch_bounds__(NWD * 64) void sdpa_decode_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    int H, int n, int m, float c_log2, int wl, int wr, int bottom_right,
    const int32_t* __restrict__ key_lens, float* __restrict__ lse, int BH, int chunk,
    float* __restrict__ part, Layout lay) {
    constexpr int NTL = KS / 16, NJ = KS / 32, NVL = KS / 8;
    constexpr int VBUF = KS * 128;  // one step of V rows in LDS
    // Per wave: two V step buffers; after the loop the first one holds the
    // wave's Oᵀ partial (64 × 16 floats = 4 KiB).
    __shared__ __attribute__((aligned(16))) char lds[NWD * 2 * VBUF];
    __shared__ float red_m[NWD][QN], red_l[NWD][QN];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int G = lane >> 4;

    // Split mode (chunk > 0, HPW = 1): workgroup g takes keys
    // [sp·chunk, (sp+1)·chunk) of head g % BH and writes its unnormalised
    // (max, sum, Oᵀ) to `part`.  Otherwise wave w serves head
    // HPW·g + w / WPH, as its (w % WPH)-th wave.
    constexpr int WPH = NWD / HPW;
    const int hw = w % WPH;
    const int bh_w = chunk > 0 ? (int)(blockIdx.x % BH) : (int)blockIdx.x * HPW + w / WPH;
    const bool hok = bh_w < BH;  // the last workgroup's heads may run out
    const int bh = hok ? bh_w : BH - 1;
    const int sp = chunk > 0 ? (int)(blockIdx.x / BH) : 0;
    const int b = bh / H;
    const int hh_b = bh - b * H;
    const uint16_t* Qh = Q + (STRIDED ? head_offset(lay.q, b, hh_b) : (long long)bh * n * D);
    const uint16_t* Kh = K + (STRIDED ? head_offset(lay.k, b, hh_b) : (long long)bh * m * D);
    const uint16_t* Vh = V + (STRIDED ? head_offset(lay.v, b, hh_b) : (long long)bh * m * D);
    const int qr = STRIDED ? lay.q.r : D, kr = STRIDED ? lay.k.r : D, vr = STRIDED ? lay.v.r : D;
    const int orr = STRIDED ? lay.o.r : D;

    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    const KeyWindow win{wl, wr, bottom_right ? L - n : 0, L};
    // Keys any query may see, in whole steps from kb; this wave's steps [s0, s1).
    int kbeg = win.lo(0), kend = win.hi(n - 1);
    if (chunk > 0) {
        kbeg = max(kbeg, sp * chunk);
        kend = min(kend, (sp + 1) * chunk);
    }
    const int kb = kbeg & ~(KS - 1);
    const int nsteps = hok && kend > kbeg ? (kend - kb + KS - 1) / KS : 0;
    const int per = (nsteps + WPH - 1) / WPH;
    const int s0 = min(nsteps, hw * per), s1 = min(nsteps, s0 + per);
    // Keys legal for every query: [flo, fhi).
    const int flo = win.lo(n - 1), fhi = win.hi(0);

    // Qᵀ as the B operand: lane holds query l16, d = 32·ks + 8·G + [0..7].
    const int q = l16;
    bf16x8 qop[2];
    if (q < n) {
        const u32x4* src = reinterpret_cast<const u32x4*>(Qh + (size_t)q * qr);
        qop[0] = __builtin_bit_cast(bf16x8, src[G]);
        qop[1] = __builtin_bit_cast(bf16x8, src[4 + G]);
    } else {
        qop[0] = qop[1] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
    // This lane's legal keys: [qlo, qhi) (empty for a padding column q >= n).
    const int qlo = q < n ? win.lo(q) : 0;
    const int qhi = q < n ? win.hi(q) : 0;

    const i32x4 rk = make_rsrc(Kh, rows_span(L, kr, D, 2));
    const i32x4 rv = make_rsrc(Vh, rows_span(L, vr, D, 2));
    const uint32_t kr2 = (uint32_t)kr * 2u, vr2 = (uint32_t)vr * 2u;  // row strides, bytes
    char* vbuf = lds + w * 2 * VBUF;
    // V loads: the i-th 1 KiB load of a step fills rows 8·i .. +7; lane ln lands
    // in LDS slot (row ln/8, position ln%8), which holds chunk (ln%8) ^ swz_f(row).
    int v_off[NVL];
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
        const int row = 8 * i + (lane >> 3);
        v_off[i] = row * (int)vr2 + (((lane & 7) ^ swz_f(row)) << 4);
    }
    // K operand of tile t, k-step ks: key k0 + 16·t + l16, d = 32·ks + 8·G.
    const int k_off = l16 * (int)kr2 + G * 16;

    // Requests step s's K (into kop) and V (into LDS buffer s & 1).  Issued
    // unconditionally, also one step past the wave's last: there the offsets
    // start at the key length, so the loads return zeros without touching
    // memory.  Every step then has the same outstanding loads, which keeps
    // the compiler's waits on K exact.  Offsets are unsigned 32-bit: the
    // sentinel L·(row stride) is below 2^31 and adds less than 64 rows, which
    // the C ABI keeps below 2^31 too, so nothing wraps (the hardware reads the
    // offset as unsigned).
    auto issue = [&](int s, bf16x8 (&kop)[NTL][2]) {
        const uint32_t row0 = s < s1 ? (uint32_t)(kb + s * KS) : (uint32_t)L;
        const uint32_t kbase = row0 * kr2, vbase = row0 * vr2;
#pragma unroll
        for (int t = 0; t < NTL; ++t)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                kop[t][ks] = __builtin_bit_cast(
                    bf16x8, sdpa_dec_buffer_load_v4i32(
                                rk, (int)(kbase + (uint32_t)(16 * t) * kr2 + (uint32_t)(k_off + 64 * ks)), 0,
                                kCachePolicyNT));
        char* dst = vbuf + (s & 1) * VBUF;
#pragma unroll
        for (int i = 0; i < NVL; ++i)
            load16_to_lds_nt(rv, dst + 8 * i * 128, (int)(vbase + (uint32_t)v_off[i]));
    };

    float mrun = -INFINITY, lrun = 0.f;
    f32x4 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One 32-key step: the next step's K and V are requested first (into the
    // other register set and LDS buffer), then this step's math.
    auto step = [&](int s, const bf16x8 (&kuse)[NTL][2], bf16x8 (&knxt)[NTL][2]) {
        const int k0 = kb + s * KS;
        // The buffer the next step fills was last read two steps ago; its
        // transpose reads have completed (their data fed that step's MFMAs).
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(s + 1, knxt);

        // Sᵀ = K · Qᵀ: register r of tile t is key k0 + 16·t + 4·G + r of query q.
        f32x4 st[NTL];
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            acc = mfma16(kuse[t][0], qop[0], acc);
            st[t] = mfma16(kuse[t][1], qop[1], acc);
        }
        if (k0 < flo || k0 + KS > fhi) {  // uniform: some key of the step is illegal somewhere
#pragma unroll
            for (int t = 0; t < NTL; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 16 * t + 4 * G + r;
                    st[t][r] = (key >= qlo && key < qhi) ? st[t][r] : -INFINITY;
                }
        }
        // Online softmax for the query column (exact running maximum).
        float mt = max2(st[0][0], st[0][1]);
        mt = max3(mt, st[0][2], st[0][3]);
#pragma unroll
        for (int t = 1; t < NTL; ++t) {
            mt = max3(mt, st[t][0], st[t][1]);
            mt = max3(mt, st[t][2], st[t][3]);
        }
        mt = quad_max(mt);
        const float mnew = fmaxf(mrun, mt);
        // mrun = −∞ (nothing legal yet) gives alpha = 0 on zeros; mnew = −∞
        // (nothing legal at all so far) keeps alpha = 1.
        const float alpha = mnew == -INFINITY ? 1.f : exp2_hw((mrun - mnew) * c_log2);
        const float mc = (mnew == -INFINITY ? 0.f : mnew) * c_log2;
        mrun = mnew;
        float p[4 * NTL];
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 4 * NTL; ++e) {
            p[e] = exp2_hw(__builtin_fmaf(st[e >> 2][e & 3], c_log2, -mc));  // −∞ → +0
            ls += p[e];
        }
        lrun = lrun * alpha + quad_sum(ls);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
        // Pᵀ as the B operand of k-step j: slots 0..3 are keys 32·j + 4·G + [0..3]
        // (tile 2·j), slots 4..7 keys 32·j + 16 + 4·G + [0..3] (tile 2·j + 1).
        bf16x8 pb[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            pb[j] = to_bf16x8(p[8 * j], p[8 * j + 1], p[8 * j + 2], p[8 * j + 3], p[8 * j + 4],
                              p[8 * j + 5], p[8 * j + 6], p[8 * j + 7]);

        // This step's V rows must have landed.  At most the next step's NVL V
        // loads may still be in flight; the count is right whatever the order
        // of the next step's K loads against them (at worst it waits longer).
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NVL) : "memory");
        // Oᵀ += Vᵀ · Pᵀ: the A operand of k-step j lists the same keys as its
        // Pᵀ, two transpose reads of 4 rows each (rows 32·j + 4·G + l16/4 and
        // + 16) of one dv column.  Written as instructions (ds_read_tr16_b64),
        // so the next step's loads stay in flight across them.
        const char* vb = vbuf + (s & 1) * VBUF;
        u32x2 vt[NJ][8];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r0 = 32 * j + 4 * G + (l16 >> 2);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const int dv0 = 16 * dt + 4 * (l16 & 3);
                vt[j][2 * dt] = ds_read_tr16_b64(vb + lds_swz(r0, dv0 >> 3) * 16 + (dv0 & 7) * 2);
                vt[j][2 * dt + 1] =
                    ds_read_tr16_b64(vb + lds_swz(r0 + 16, dv0 >> 3) * 16 + (dv0 & 7) * 2);
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) tr_wait(vt[j]);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const u32x4 a = {vt[j][2 * dt][0], vt[j][2 * dt][1], vt[j][2 * dt + 1][0],
                                 vt[j][2 * dt + 1][1]};
                o[dt] = mfma16(__builtin_bit_cast(bf16x8, a), pb[j], o[dt]);
            }
    };

    // Two register sets for K, used alternately (no copies across iterations).
    bf16x8 kA[NTL][2], kB[NTL][2];
    issue(s0, kA);
    for (int s = s0; s < s1; s += 2) {
        step(s, kA, kB);
        if (s + 1 >= s1) break;
        step(s + 1, kB, kA);
    }

    // ---- merge the four waves' partials.  Register r of o[dt] is dv = 16·dt
    // + 4·G + r of query q; the wave's Oᵀ goes to its own first V buffer.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    float* po = reinterpret_cast<float*>(vbuf);  // [dv][QN]
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) po[(16 * dt + 4 * G + r) * QN + q] = o[dt][r];
    if (G == 0) {
        red_m[w][q] = mrun;
        red_l[w][q] = lrun;
    }
    __syncthreads();
    // The threads of head hh (NWD·64 / HPW of them) finish it: thread t takes
    // query t % 16 and DPT = 4·HPW dims from dv fd on.
    constexpr int TPH = NWD * 64 / HPW, DPT = 4 * HPW;
    const int hh = tid / TPH, tl = tid % TPH;
    const int fq = tl & (QN - 1);
    const int fd = DPT * (tl >> 4);
    const int bh_t = chunk > 0 ? bh : (int)blockIdx.x * HPW + hh;  // this thread's head
    const int b_t = bh_t / H;
    uint16_t* Oh_t = O + (STRIDED ? head_offset(lay.o, b_t, bh_t - b_t * H) : (long long)bh_t * n * D);
    if (fq < n && bh_t < BH) {
        const int u0 = hh * WPH;
        float mx = red_m[u0][fq];
#pragma unroll
        for (int u = 1; u < WPH; ++u) mx = fmaxf(mx, red_m[u0 + u][fq]);
        const float mcx = (mx == -INFINITY ? 0.f : mx) * c_log2;
        float lt = 0.f;
        float acc[DPT];
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
#pragma unroll
        for (int u = 0; u < WPH; ++u) {
            // a wave with no legal key (max −∞) contributes exactly nothing
            const float mu = red_m[u0 + u][fq];
            const float sc = mu == -INFINITY ? 0.f : exp2_hw(mu * c_log2 - mcx);
            lt += sc * red_l[u0 + u][fq];
            const float* pu = reinterpret_cast<const float*>(lds + (u0 + u) * 2 * VBUF);
#pragma unroll
            for (int e = 0; e < DPT; ++e) acc[e] += sc * pu[(fd + e) * QN + fq];
        }
        if (chunk > 0) {
            // [m, l, -, -, O(64)] of query fq, split sp: O unnormalised, l
            // against max m (68 floats, so that O stays 16-byte aligned)
            float* pp = part + ((size_t)(sp * BH + bh) * n + fq) * PREC;
            if (fd == 0) {
                pp[0] = mx;
                pp[1] = lt;
            }
            *reinterpret_cast<f32x4*>(pp + 4 + fd) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            return;
        }
        // no legal key ⇒ zero row; a NaN sum (NaN legal inputs) stays NaN
        const float inv = lt != 0.f ? 1.f / lt : 0.f;
        // ln Σ e^(scale·s) = (mcx + log2 lt)·ln 2: −∞ for a row with no legal key
        if (lse && fd == 0) lse[(size_t)bh_t * n + fq] = (mcx + log2f(lt)) * 0.6931471805599453f;
#pragma unroll
        for (int c = 0; c < DPT; c += 4) {
            bf16x4 ov;
            ov[0] = (__bf16)(acc[c + 0] * inv);
            ov[1] = (__bf16)(acc[c + 1] * inv);
            ov[2] = (__bf16)(acc[c + 2] * inv);
            ov[3] = (__bf16)(acc[c + 3] * inv);
            *reinterpret_cast<bf16x4*>(Oh_t + (size_t)fq * orr + fd + c) = ov;
        }
    }
}

}  // namespace

// Combine the splits of each (head, query): the usual rescale to the largest
// maximum.  One workgroup per (head, query); thread t takes dims
// 4·(t % 16) .. +3 of the splits t / 16, t / 16 + 16, ..., and the sixteen
// partial merges are combined through LDS at the end.
__global__ __launch_bounds__(NWD * 64) void sdpa_decode_merge_bf16(
    const float* __restrict__ part, uint16_t* __restrict__ O, float* __restrict__ lse, int BH, int H,
    int n, int nsplit, float c_log2, Strides os) {
    constexpr int SL = NWD * 64 / 16;  // split slots
    const int bh = blockIdx.x / n, fq = blockIdx.x % n;
    const int fd = 4 * (threadIdx.x & 15);
    const int sl = threadIdx.x >> 4;
    const size_t stride = (size_t)BH * n * PREC;  // from one split to the next
    const float* p0 = part + ((size_t)bh * n + fq) * PREC;
    // Four splits per round: all their loads are issued before any use.
    float mx = -INFINITY, lt = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = sl; s0 < nsplit; s0 += 4 * SL) {
        float ms[4], ls[4];
        f32x4 os[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int sp = s0 + u * SL;
            const bool ok = sp < nsplit;
            const float* ps = p0 + (size_t)(ok ? sp : 0) * stride;
            ms[u] = ok ? ps[0] : -INFINITY;
            ls[u] = ok ? ps[1] : 0.f;
            os[u] = ok ? *reinterpret_cast<const f32x4*>(ps + 4 + fd) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        float mnew = mx;
#pragma unroll
        for (int u = 0; u < 4; ++u) mnew = fmaxf(mnew, ms[u]);
        const float mc = (mnew == -INFINITY ? 0.f : mnew) * c_log2;
        // the old partial and a split with no legal key (max −∞) scale by exactly 0
        const float so = mx == -INFINITY ? 0.f : exp2_hw(mx * c_log2 - mc);
        lt *= so;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= so;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float sc = ms[u] == -INFINITY ? 0.f : exp2_hw(ms[u] * c_log2 - mc);
            lt += sc * ls[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += sc * os[u][e];
        }
        mx = mnew;
    }
    __shared__ float red_m[SL], red_l[SL];
    __shared__ f32x4 red_o[SL][16];
    if (fd == 0) {
        red_m[sl] = mx;
        red_l[sl] = lt;
    }
    red_o[sl][fd >> 2] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    __syncthreads();
    if (sl != 0) return;
    float mt = red_m[0];
#pragma unroll
    for (int i = 1; i < SL; ++i) mt = fmaxf(mt, red_m[i]);
    const float mcx = (mt == -INFINITY ? 0.f : mt) * c_log2;
    float ltot = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < SL; ++i) {
        const float sc = red_m[i] == -INFINITY ? 0.f : exp2_hw(red_m[i] * c_log2 - mcx);
        ltot += sc * red_l[i];
        const f32x4 x = red_o[i][fd >> 2];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += sc * x[e];
    }
    // no legal key ⇒ zero row; a NaN sum (NaN legal inputs) stays NaN
    const float inv = ltot != 0.f ? 1.f / ltot : 0.f;
    if (lse && fd == 0) lse[(size_t)bh * n + fq] = (mcx + log2f(ltot)) * 0.6931471805599453f;
    bf16x4 ov;
    ov[0] = (__bf16)(o[0] * inv);
    ov[1] = (__bf16)(o[1] * inv);
    ov[2] = (__bf16)(o[2] * inv);
    ov[3] = (__bf16)(o[3] * inv);
    *reinterpret_cast<bf16x4*>(O + head_offset(os, bh / H, bh % H) + (size_t)fq * os.r + fd) = ov;
}

// Keys per split: 1024 (eight 32-key steps per wave) when that already gives
// 1024 workgroups (four per CU, what their LDS allows); with fewer heads the
// pieces shrink, down to 256 keys, towards that count.  Splitting pays when a
// head's keys are long and either the heads are few (one workgroup per head
// leaves most CUs idle) or their lengths differ.  (2048- and 4096-key pieces
// measured slower on ragged 2k..8k caches with 256 heads.)
int decode_chunk(long long BH, int m) {
    int c = 1024;
    while (c > 256 && BH * ((m + c - 1) / c) < 1024) c /= 2;
    return c;
}

size_t decode_split_bytes(int B, int H, int n, int m) {
    // A few queries against more keys than the sentence-length kernel takes,
    // spread over at least two pieces.
    if (n > QN || m <= 64) return 0;
    const int chunk = decode_chunk((long long)B * H, m);
    const int ns = (m + chunk - 1) / chunk;
    if (ns < 2) return 0;
    return (size_t)ns * B * H * n * PREC * sizeof(float);
}

bool decode_bf16_fits(const Args& a) {
    if (a.n > QN || a.m <= 64) return false;
    // One workgroup per head needs enough heads to give every CU work; with a
    // workspace the split mode gives every piece of keys its own workgroup,
    // so any number of heads (a single sequence's decoder step included) fits.
    if ((long long)a.B * a.H >= 256) return true;
    const size_t need = decode_split_bytes(a.B, a.H, a.n, a.m);
    return a.work && need > 0 && a.work_bytes >= need;
}

hipError_t launch_bf16_decode(const Args& a, hipStream_t stream) {
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    const int BH = a.B * a.H;
    const size_t need = decode_split_bytes(a.B, a.H, a.n, a.m);
    if (a.work && need > 0 && a.work_bytes >= need) {
        const int chunk = decode_chunk(BH, a.m);
        const int ns = (a.m + chunk - 1) / chunk;
        const auto split_kernel = a.strided ? sdpa_decode_bf16<32, 1, true> : sdpa_decode_bf16<32, 1, false>;
        hipLaunchKernelGGL(split_kernel, dim3(BH * ns), dim3(NWD * 64), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (uint16_t*)a.out, a.H, a.n, a.m, c_log2, a.wl, a.wr, a.bottom_right,
                           a.key_lens, a.lse, BH, chunk, (float*)a.work, a.lay);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(sdpa_decode_merge_bf16, dim3(BH * a.n), dim3(NWD * 64), 0, stream,
                           (const float*)a.work, (uint16_t*)a.out, a.lse, BH, a.H, a.n, ns, c_log2, a.lay.o);
        return hipGetLastError();
    }
    // 32-key steps.  64-key steps (twice the bytes per request round trip)
    // measured no faster on 2k..8k-key caches and slower on full 8k caches.
    // Short caches and many heads: two heads per workgroup (two waves each), so
    // that every head is resident at once (four workgroups fit per CU).  On
    // beam-search steps against ≤ 128 keys this measured 11.4 vs 12.4 µs;
    // long caches need all four waves on one head (113 vs 66 µs at 2k..8k).
    if (a.m <= 256 && BH >= 1024) {
        const auto kernel2 = a.strided ? sdpa_decode_bf16<32, 2, true> : sdpa_decode_bf16<32, 2, false>;
        hipLaunchKernelGGL(kernel2, dim3((BH + 1) / 2), dim3(NWD * 64), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (uint16_t*)a.out, a.H, a.n, a.m, c_log2, a.wl, a.wr, a.bottom_right,
                           a.key_lens, a.lse, BH, 0, nullptr, a.lay);
    } else {
        const auto kernel1 = a.strided ? sdpa_decode_bf16<32, 1, true> : sdpa_decode_bf16<32, 1, false>;
        hipLaunchKernelGGL(kernel1, dim3(BH), dim3(NWD * 64), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (uint16_t*)a.out, a.H, a.n, a.m, c_log2, a.wl, a.wr, a.bottom_right,
                           a.key_lens, a.lse, BH, 0, nullptr, a.lay);
    }
    return hipGetLastError();
}

}  // namespace sdpa
