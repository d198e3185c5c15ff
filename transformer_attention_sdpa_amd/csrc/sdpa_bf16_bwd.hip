// Gradient of scaled dot-product attention on gfx950 (bf16 in and out, fp32
// accumulation).
//
// The pages print only the forward pass, Eq. (1) (《精读 Attention Is All You
// Need：原始 Transformer 论文》, "缩放点积注意力：点积为什么要缩放";
// 《Attention Is All You Need：注意力就是你所需要的一切》 §3.2.1), and train the
// model through it.  By the chain rule, with s = scale·q·k, P = softmax(S)
// row-wise and O = P V:
//
//   dV = Pᵀ dO,   dP = dO Vᵀ,   dS = P ∘ (dP − D),   D_i = Σ_j P_ij dP_ij = dO_i · O_i,
//   dQ = scale · dS K,   dK = scale · dSᵀ Q.
//
// P is recomputed tile by tile from the forward pass's per-row log-sum-exp,
// P_ij = exp(s_ij − lse_i), so no n×m matrix is ever stored.  Two launches,
// neither with atomics (the result is bitwise deterministic):
//
//   1. sdpa_bwd_dq_bf16, one workgroup per block of 32·NW queries: computes
//      D_i and lse_i·log2 e for its rows (written to the workspace for launch
//      2), then streams the K/V tiles its queries may see:
//        Sᵀ = K Qᵀ, dPᵀ = V dOᵀ (A from LDS rows, B = Qᵀ, dOᵀ in VGPRs),
//        dSᵀ = Pᵀ ∘ (dPᵀ − D),  dQᵀ += Kᵀ dSᵀ (A via LDS transpose reads).
//   2. sdpa_bwd_dkdv_bf16, one workgroup per block of 32·NW keys: streams the
//      Q/dO tiles of the queries that may see them:
//        S = Q Kᵀ, dP = dO Vᵀ (A from LDS rows, B = Kᵀ, Vᵀ in VGPRs),
//        dVᵀ += dOᵀ P,  dKᵀ += Qᵀ dS (A via LDS transpose reads).
//
// Every product is v_mfma_f32_32x32x16_bf16 with the accumulator of one
// product (lane = one column, 16 rows in groups of 4) serving directly as the
// B operand of the next: the contraction index then runs in the permuted
// order 16·j + 4·hf + [0..3], 16·j + 8 + 4·hf + [0..3] for k-step j, and the
// transpose reads fetch the A operand in that same order.  P and dS are
// rounded to bf16 for their products, as in the forward pass.
//
// LDS reads are written as instructions (ds_read_b128, ds_read_b64_tr_b16)
// with explicit lgkmcnt waits: through plain loads or the builtins the
// compiler would wait for the next tile's buffer_load … lds, which is in
// flight during the current tile's math, before every read.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int BT = 64;                          // rows per LDS tile
template <int D>
constexpr int tile_bytes() { return BT * D * 2; }

// 16-byte chunk position of chunk c of row r in a tile of D/8 chunks per row,
// XOR-swizzled so that 16 consecutive rows read at one chunk fall on distinct
// banks of the 256-byte LDS pass (64-byte rows share a pass four at a time,
// 256-byte rows fill it alone); for D = 64 it is lds_swz.  At D = 128 the
// row's low two bits select the 4-chunk group and the next two the chunk in
// it, so that the transpose reads (rows 4·G' + [0..3] at four consecutive
// chunks) spread over all banks too.
template <int D>
__device__ __forceinline__ int bswz(int r, int c) {
    if constexpr (D == 32) return r * 4 + (c ^ ((r >> 2) & 3));
    else if constexpr (D == 128) return r * 16 + (c ^ (((r & 3) << 2) | ((r >> 2) & 3)));
    else return lds_swz(r, c);
}
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t a) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
__device__ __forceinline__ u32x2 ds_read_tr(uint32_t a) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
// Wait for every LDS read of this wave; the results pass through the empty
// asm after the wait, so no use of them can move above it.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4 (&x)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x2 (&x)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}

// Per-lane LDS offsets inside one 64-row tile of width D (16-byte chunk c of
// row r at bswz<D>(r, c)), shared by the kernels.
template <int D>
struct TileAddr {
    int row[D / 16];    // 16-byte A operand of k-step ks: row l32, chunk 2·ks + hf
    int tr[D / 32][2];  // transpose reads of k-step 0: [32-column block dt][rows +0 / +8]
    __device__ void init(int lane) {
        const int l32 = lane & 31, hf = lane >> 5, gi = lane & 15;
        // (rows l32 and l32 + 32 share the swizzle of every width)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) row[ks] = bswz<D>(l32, 2 * ks + hf) * 16;
        // Rows 4·hf + gi/4 (+ 8) of k-step 0; k-step j adds 16·j rows, which
        // leaves the swizzle of every width unchanged.
        const int r0 = 4 * hf + (gi >> 2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int c0 = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
            tr[dt][0] = bswz<D>(r0, c0 >> 3) * 16 + (c0 & 7) * 2;
            tr[dt][1] = bswz<D>(r0 + 8, c0 >> 3) * 16 + (c0 & 7) * 2;
        }
    }
};

// k-step j of a two-tile accumulator pair as a bf16 B operand: tile j/2,
// registers 8·(j%2) .. +7.
__device__ __forceinline__ bf16x8 pack_step(const f32x16 (&x)[2], int j) {
    const int t = j >> 1, b = 8 * (j & 1);
    return to_bf16x8(x[t][b], x[t][b + 1], x[t][b + 2], x[t][b + 3], x[t][b + 4], x[t][b + 5],
                     x[t][b + 6], x[t][b + 7]);
}

// acc[dt] += Aᵀ · B over one 64-row tile: A is the tile (rows = contraction
// index, columns = the 64 output rows), fetched with transpose reads in the
// permuted contraction order; b[j] is k-step j of the B operand.
template <int D>
__device__ __forceinline__ void tr_product(uint32_t tile, const TileAddr<D>& ta, const bf16x8 (&b)[4],
                                           f32x16 (&acc)[D / 32]) {
    constexpr int DT = D / 32;
    u32x2 a[8 * DT];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            a[(j * DT + dt) * 2] = ds_read_tr(tile + ta.tr[dt][0] + j * 16 * D * 2);
            a[(j * DT + dt) * 2 + 1] = ds_read_tr(tile + ta.tr[dt][1] + j * 16 * D * 2);
        }
    lds_wait(a);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const u32x2 lo = a[(j * DT + dt) * 2], hi = a[(j * DT + dt) * 2 + 1];
            const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
            acc[dt] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, v), b[j], acc[dt]);
        }
}

// s[t] = A_t · B (and, with TWO, p[t] = A'_t · B') for the two 32-row halves
// t of tiles A, A' (rows from LDS) against B, B' (k = D dims, in VGPRs).
template <int D, bool TWO>
__device__ __forceinline__ void row_products(uint32_t ta_, uint32_t tb_, const TileAddr<D>& ta,
                                             const bf16x8 (&b)[D / 16], const bf16x8 (&b2)[D / 16],
                                             f32x16 (&s)[2], f32x16 (&p)[2]) {
    constexpr int KS = D / 16, NA = TWO ? 2 : 1;
    u32x4 a[NA * 2 * KS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            a[t * KS + ks] = ds_read_b128(ta_ + ta.row[ks] + t * 32 * D * 2);
            if constexpr (TWO) a[2 * KS + t * KS + ks] = ds_read_b128(tb_ + ta.row[ks] + t * 32 * D * 2);
        }
    lds_wait(a);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[t][i] = 0.f;
            if constexpr (TWO) p[t][i] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[t] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, a[t * KS + ks]), b[ks], s[t]);
            if constexpr (TWO)
                p[t] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, a[2 * KS + t * KS + ks]), b2[ks], p[t]);
        }
    }
}

// This lane's 16-byte operand chunks of one D-wide row (dims 16·ks + 8·hf
// + [0..7]), zeros if the row is out of range.
template <int D>
__device__ __forceinline__ void load_row_operand(const uint16_t* rowp, bool ok, int hf, bf16x8 (&x)[D / 16]) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        x[ks] = ok ? __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4*>(rowp)[2 * ks + hf])
                   : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
}

// Store a transposed accumulator pair (register i of acc[dt] is column
// 32·dt + 8·(i/4) + 4·hf + i%4 of this lane's row) times `mul` as bf16.
template <int D>
__device__ __forceinline__ void store_rowT(uint16_t* dst, const f32x16 (&acc)[D / 32], int hf, float mul) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            bf16x4 o;
            o[0] = (__bf16)(acc[dt][4 * i4 + 0] * mul);
            o[1] = (__bf16)(acc[dt][4 * i4 + 1] * mul);
            o[2] = (__bf16)(acc[dt][4 * i4 + 2] * mul);
            o[3] = (__bf16)(acc[dt][4 * i4 + 3] * mul);
            *reinterpret_cast<bf16x4*>(dst + 32 * dt + 8 * i4 + 4 * hf) = o;
        }
}

// Store 32 output rows of width D through a wave-private LDS area of 64·D
// bytes: the transposed accumulators (register i of acc[dt] is column 32·dt +
// 8·(i/4) + 4·hf + i%4 of row l32) go in as bf16 times `mul`, and come out 16
// bytes a lane, so that each store instruction writes whole rows instead of
// 32 scattered 8-byte pieces.  Rows at or past `nrows` are not written.
template <int D>
__device__ __forceinline__ void store_rows_lds(char* area, const f32x16 (&acc)[D / 32], int lane, float mul,
                                               uint16_t* dst, int nrows) {
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int col = 32 * dt + 8 * i4 + 4 * hf;
            bf16x4 o;
            o[0] = (__bf16)(acc[dt][4 * i4 + 0] * mul);
            o[1] = (__bf16)(acc[dt][4 * i4 + 1] * mul);
            o[2] = (__bf16)(acc[dt][4 * i4 + 2] * mul);
            o[3] = (__bf16)(acc[dt][4 * i4 + 3] * mul);
            *reinterpret_cast<bf16x4*>(area + bswz<D>(l32, col >> 3) * 16 + (col & 7) * 2) = o;
        }
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
        const int row = (64 / CPR) * k + lane / CPR, c = lane % CPR;
        const u32x4 x = *reinterpret_cast<const u32x4*>(area + bswz<D>(row, c) * 16);
        if (row < nrows) store16_nt(dst + (size_t)row * D + 8 * c, x);
    }
}

// Copy rows [r0, r0 + 64) of a [len, D] bf16 tensor into an LDS tile; rows
// at or past `len` arrive as zeros.  Wave w of NW issues its share of the
// tile's 1 KiB loads; lane ln lands in (row ln/CPR, position ln%CPR) of the
// load's rows, which holds the chunk whose swizzled position that is.
template <int D, int NW>
__device__ __forceinline__ void load_tile(char* lds_tile, const uint16_t* base, int r0, int len, int w,
                                          int lane) {
    constexpr int CPR = D / 8, LOADS = tile_bytes<D>() / 1024 / NW, RPL = 1024 / (D * 2);
    const int left = len - r0;
    const i32x4 rs = make_rsrc(base + (size_t)r0 * D, (uint32_t)(left > 0 ? left : 0) * (D * 2));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int blk = w * LOADS + i;
        const int row = RPL * blk + lane / CPR;
        const int chunk = bswz<D>(row, lane % CPR) - row * CPR;  // XOR is its own inverse
        load16_to_lds(rs, lds_tile + blk * 1024, row * D * 2 + chunk * 16);
    }
}

// ---------------------------------------------------------------------------
// Launch 1: dQ (and D, lse·log2 e for launch 2).

// DROP: attention dropout of the forward pass with keep-bit words [BH, n, ⌈m/32⌉]:
// dP = (dO Vᵀ) ∘ Z · keep_scale.
template <int D, int NW, bool DROP>
__global__ __launch_bounds__(NW * 64) void sdpa_bwd_dq_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    uint16_t* __restrict__ dQ, float* __restrict__ ws_d, float* __restrict__ ws_l,
    int BH, int H, int n, int m, float scale, float c_log2, int wl, int wr, int bottom_right,
    const int32_t* __restrict__ key_lens, int nqb, const uint32_t* __restrict__ keep, float keep_scale) {
    constexpr int TB = tile_bytes<D>(), KS = D / 16, DT = D / 32;
    __shared__ __attribute__((aligned(1024))) char lds[2 * 2 * TB];  // [buf][K | V]
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;

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
    // This wave's queries: keys [wlo, whi) are needed, [flo, fhi) legal for all.
    const int wq0 = q0 + 32 * w;
    const int wlast = min(wq0 + 32, n) - 1;
    const bool wact = wlast >= wq0;
    const int wlo = wact ? win.lo(wq0) : 0, whi = wact ? win.hi(wlast) : 0;
    const int flo = wact ? win.lo(wlast) : 0, fhi = wact ? win.hi(wq0) : 0;

    const size_t qbase = (size_t)bh * n * D, kvbase = (size_t)bh * m * D;
    const int qrow = wq0 + l32;
    const bool qok = qrow < n;
    bf16x8 qop[KS], dop[KS];
    load_row_operand<D>(Q + qbase + (size_t)qrow * D, qok, hf, qop);
    load_row_operand<D>(dO + qbase + (size_t)qrow * D, qok, hf, dop);
    // D_i = dO_i · O_i over this lane's half of the dims, then the other half-wave's.
    float dsum;
    {
        bf16x8 oop[KS];
        load_row_operand<D>(O + qbase + (size_t)qrow * D, qok, hf, oop);
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)dop[ks][e], (float)oop[ks][e], acc);
        dsum = half_swap_sum(acc);
    }
    // P = 2^(s·c − lc); a row with no legal key (lse = −∞) gets lc = +∞, P = 0.
    const float lr = qok ? lse[(size_t)bh * n + qrow] : 0.f;
    const float lc = lr == -INFINITY ? INFINITY : lr * LOG2E;
    if (qok && hf == 0) {
        ws_d[(size_t)bh * n + qrow] = dsum;
        ws_l[(size_t)bh * n + qrow] = lc;
    }

    // Dropout: this lane's row of keep words (rows past n read row n − 1; their
    // dQ is not stored).
    const int kwords = (m + 31) >> 5;
    const uint32_t* krow = DROP ? keep + ((size_t)bh * n + min(qrow, n - 1)) * kwords : nullptr;

    TileAddr<D> ta;
    ta.init(lane);
    const uint32_t l0 = lds_u32(lds);
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

    auto issue = [&](int t, int buf) {
        load_tile<D, NW>(lds + buf * 2 * TB, K + kvbase, t * BT, L, w, lane);
        load_tile<D, NW>(lds + buf * 2 * TB + TB, V + kvbase, t * BT, L, w, lane);
    };
    if (tend > tbeg) issue(tbeg, 0);
    wait_vmem();
    __syncthreads();
    for (int t = tbeg; t < tend; ++t) {
        const int buf = (t - tbeg) & 1;
        if (t + 1 < tend) issue(t + 1, buf ^ 1);
        const int k0 = t * BT;
        if (k0 < whi && k0 + BT > wlo) {  // uniform: some query of the wave sees the tile
            const uint32_t sk = l0 + buf * 2 * TB, sv = sk + TB;
            uint32_t kw[2] = {0u, 0u};  // keep words of keys k0.. and k0 + 32..
            if constexpr (DROP) {
                const int w0 = k0 >> 5;
                kw[0] = w0 < kwords ? krow[w0] : 0u;
                kw[1] = w0 + 1 < kwords ? krow[w0 + 1] : 0u;
            }
            f32x16 s[2], dp[2];
            row_products<D, true>(sk, sv, ta, qop, dop, s, dp);
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
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = exp2_hw(__builtin_fmaf(s[kt][i], c_log2, -lc));
                    float g = dp[kt][i];
                    if constexpr (DROP)
                        g = (kw[kt] >> (8 * (i >> 2) + 4 * hf + (i & 3))) & 1u ? g * keep_scale : 0.f;
                    s[kt][i] = p * (g - dsum);  // dSᵀ
                }
            bf16x8 db[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) db[j] = pack_step(s, j);
            tr_product<D>(sk, ta, db, acc);  // dQᵀ += Kᵀ dSᵀ
        }
        wait_vmem();
        __syncthreads();
    }
    if (qok) store_rowT<D>(dQ + qbase + (size_t)qrow * D, acc, hf, scale);
}

// ---------------------------------------------------------------------------
// Launch 2: dK, dV.

// Queries that may see key j form the interval [qa, qb) (the legal keys of a
// query, [lo_i, hi_i), move right with i).  Keys at or past L see none.
struct QueryRange {
    int wl, wr, shift, L, n;
    __device__ __forceinline__ int qa(int j) const {
        if (j >= L) return 0;
        if (wr < 0) return 0;
        const long long c = (long long)j - shift - wr;  // hi_i > j  ⇔  i ≥ j − shift − wr
        return c <= 0 ? 0 : (c >= n ? n : (int)c);
    }
    __device__ __forceinline__ int qb(int j) const {
        if (j >= L) return 0;
        if (wl < 0) return n;
        const long long c = (long long)j - shift + wl + 1;  // lo_i ≤ j  ⇔  i ≤ j − shift + wl
        return c <= 0 ? 0 : (c >= n ? n : (int)c);
    }
};

// DV, DK: which gradients this launch forms (both, for D <= 64; at D = 128 one
// launch each keeps the accumulators within the register file).
// DROP: attention dropout as in the dQ kernel; dVᵀ += dOᵀ (P ∘ Z · keep_scale).
template <int D, int NW, bool DV, bool DK, bool DROP>
__global__ __launch_bounds__(NW * 64) void sdpa_bwd_dkdv_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ ws_d, const float* __restrict__ ws_l,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int BH, int H, int n, int m, float scale, float c_log2, int wl, int wr, int bottom_right,
    const int32_t* __restrict__ key_lens, const uint32_t* __restrict__ keep, float keep_scale) {
    // [buf][Q tile | dO tile | lse·log2 e (64 floats) | D (64 floats) | with
    // DROP, per wave the keep words of its 32 keys for the tile's 64 queries]
    constexpr int TB = tile_bytes<D>(), KS = D / 16, DT = D / 32;
    constexpr int STAGE = 2 * TB + 512 + (DROP ? NW * 256 : 0);
    __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;

    // Earliest key blocks first (seen by the most queries under a causal mask).
    const int g = blockIdx.x;
    const int bh = g % BH;
    const int k0 = (g / BH) * 32 * NW;
    const int b = bh / H;
    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    const QueryRange qr{wl, wr, bottom_right ? L - n : 0, L, n};
    // Queries [qbeg, qend) see some key of the block.
    const int klast = min(k0 + 32 * NW, L) - 1;
    const int qbeg = klast >= k0 ? qr.qa(k0) : 0;
    const int qend = klast >= k0 ? qr.qb(klast) : 0;
    const int tbeg = qbeg / BT;
    const int tend = qend > qbeg ? (qend + BT - 1) / BT : tbeg;
    // This wave's keys: queries [wqa, wqb) needed, [fqa, fqb) see all of them.
    const int wk0 = k0 + 32 * w;
    const int wlast = min(wk0 + 32, L) - 1;
    const bool wact = wlast >= wk0;
    const int wqa = wact ? qr.qa(wk0) : 0, wqb = wact ? qr.qb(wlast) : 0;
    // a wave holding keys past L never has a tile legal for all of them
    const bool wfull = wact && wk0 + 31 < L;
    const int fqa = wfull ? qr.qa(wlast) : 0, fqb = wfull ? qr.qb(wk0) : 0;

    const size_t qbase = (size_t)bh * n * D, kvbase = (size_t)bh * m * D;
    const int kwords = (m + 31) >> 5;
    const int key = wk0 + l32;
    // Kᵀ, Vᵀ as B operands; keys at or past L are zeros (their rows may hold
    // anything), so their logits are masked and their dS is exactly 0.
    bf16x8 kop[KS], vop[KS];
    load_row_operand<D>(K + kvbase + (size_t)key * D, key < L, hf, kop);
    if constexpr (DK) load_row_operand<D>(V + kvbase + (size_t)key * D, key < L, hf, vop);
    const int ka = qr.qa(key), kb = qr.qb(key);

    TileAddr<D> ta;
    ta.init(lane);
    const uint32_t l0 = lds_u32(lds);
    f32x16 dka[DK ? DT : 1], dva[DV ? DT : 1];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int dt = 0; dt < (DK ? DT : 1); ++dt) dka[dt][i] = 0.f;
#pragma unroll
        for (int dt = 0; dt < (DV ? DT : 1); ++dt) dva[dt][i] = 0.f;
    }

    auto issue = [&](int t, int buf) {
        char* st = lds + buf * STAGE;
        load_tile<D, NW>(st, Q + qbase, t * BT, n, w, lane);
        load_tile<D, NW>(st + TB, dO + qbase, t * BT, n, w, lane);
        if (w == 0) {  // 64 floats each: one dword per lane
            const int left = n - t * BT;
            const uint32_t nb = (uint32_t)(left > 0 ? left : 0) * 4u;
            const i32x4 rl = make_rsrc(ws_l + (size_t)bh * n + t * BT, nb);
            const i32x4 rd = make_rsrc(ws_d + (size_t)bh * n + t * BT, nb);
            sdpa_llvm_buffer_load_lds(rl, (__attribute__((address_space(3))) void*)(st + 2 * TB), 4,
                                      lane * 4, 0, 0, 0);
            sdpa_llvm_buffer_load_lds(rd, (__attribute__((address_space(3))) void*)(st + 2 * TB + 256),
                                      4, lane * 4, 0, 0, 0);
        }
        if constexpr (DROP) {  // word wk0/32 of query rows t·BT + lane, zeros past n
            // (a wave whose keys start at or past m has no word: nothing is read)
            const int left = n - t * BT;
            const uint32_t nb = left > 0 && wk0 < m ? (uint32_t)(((left < BT ? left : BT) - 1) * kwords + 1) * 4u
                                                    : 0u;
            const i32x4 rk = make_rsrc(keep + ((size_t)bh * n + t * BT) * kwords + (wk0 < m ? wk0 >> 5 : 0), nb);
            sdpa_llvm_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(st + 2 * TB + 512 + w * 256),
                                      4, lane * kwords * 4, 0, 0, 0);
        }
    };
    if (tend > tbeg) issue(tbeg, 0);
    wait_vmem();
    __syncthreads();
    for (int t = tbeg; t < tend; ++t) {
        const int buf = (t - tbeg) & 1;
        if (t + 1 < tend) issue(t + 1, buf ^ 1);
        const int t0 = t * BT;
        if (t0 < wqb && t0 + BT > wqa) {  // uniform: some query of the tile sees a key of the wave
            const uint32_t sq = l0 + buf * STAGE, sd = sq + TB;
            f32x16 s[2], dp[2];
            row_products<D, DK>(sq, sd, ta, kop, vop, s, dp);
            // Register i of s[qh] is query t0 + 32·qh + 8·(i/4) + 4·hf + i%4.
            if (t0 < fqa || t0 + BT > fqb) {
                const int llo = ka - t0 - 4 * hf, lhi = kb - t0 - 4 * hf;
#pragma unroll
                for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int off = 32 * qh + 8 * (i >> 2) + (i & 3);
                        s[qh][i] = (off >= llo && off < lhi) ? s[qh][i] : -INFINITY;
                    }
            }
            // lse·log2 e and D of those queries: four consecutive floats per
            // group of four registers.
            u32x4 lv[8];
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const uint32_t off = (uint32_t)(32 * qh + 8 * gq + 4 * hf) * 4u;
                    lv[4 * qh + gq] = ds_read_b128(sq + 2 * TB + off);
                }
            lds_wait(lv);
            u32x4 dv4[8];
            if constexpr (DK) {
#pragma unroll
                for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const uint32_t off = (uint32_t)(32 * qh + 8 * gq + 4 * hf) * 4u;
                        dv4[4 * qh + gq] = ds_read_b128(sq + 2 * TB + 256 + off);
                    }
                lds_wait(dv4);
            }
            // Dropout: the keep words of those queries for this wave's keys;
            // bit i of zb[qh] is bit l32 (this lane's key) of register i's query.
            uint32_t zb[2] = {0u, 0u};
            if constexpr (DROP) {
                u32x4 kq[8];
#pragma unroll
                for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const uint32_t off = (uint32_t)(32 * qh + 8 * gq + 4 * hf) * 4u;
                        kq[4 * qh + gq] = ds_read_b128(sq + 2 * TB + 512 + w * 256 + off);
                    }
                lds_wait(kq);
#pragma unroll
                for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                    for (int i = 0; i < 16; ++i) zb[qh] |= ((kq[4 * qh + (i >> 2)][i & 3] >> l32) & 1u) << i;
            }
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float lc = __uint_as_float(lv[4 * qh + (i >> 2)][i & 3]);
                    const float p = exp2_hw(__builtin_fmaf(s[qh][i], c_log2, -lc));
                    float pd = p;  // the weight that multiplied the value (P ∘ Z · c)
                    float g = DK ? dp[qh][i] : 0.f;
                    if constexpr (DROP) {
                        const bool z = (zb[qh] >> i) & 1u;
                        pd = z ? p * keep_scale : 0.f;
                        g = z ? g * keep_scale : 0.f;
                    }
                    s[qh][i] = pd;
                    if constexpr (DK) {
                        const float dd = __uint_as_float(dv4[4 * qh + (i >> 2)][i & 3]);
                        dp[qh][i] = p * (g - dd);  // dS
                    }
                }
            if constexpr (DV) {
                bf16x8 pb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) pb[j] = pack_step(s, j);
                tr_product<D>(sd, ta, pb, dva);  // dVᵀ += dOᵀ P
            }
            if constexpr (DK) {
                bf16x8 db[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) db[j] = pack_step(dp, j);
                tr_product<D>(sq, ta, db, dka);  // dKᵀ += Qᵀ dS
            }
        }
        wait_vmem();
        __syncthreads();
    }
    if (key < m) {
        if constexpr (DK) store_rowT<D>(dK + kvbase + (size_t)key * D, dka, hf, scale);
        if constexpr (DV) store_rowT<D>(dV + kvbase + (size_t)key * D, dva, hf, 1.f);
    }
}

// ---------------------------------------------------------------------------
// Sentence length (n, m ≤ 64): one workgroup per head, one launch.  The
// head's Q, dO, K and V (64·D·2 bytes each) are copied into LDS once; waves 2
// and 3 take the dQ role for queries 0..31 and 32..63 (and first publish D
// and lse·log2 e of their rows through LDS), waves 0 and 1 the dK/dV role for
// keys 0..31 and 32..63.  Each role is one tile of the two kernels above.
// DROP: the head's keep words (at most 64 rows of 2) are staged in LDS as
// [word][query], and dP, and the weights of dV, take the mask and factor as
// in the two kernels above.

template <int D, bool DROP>
__global__ __launch_bounds__(256) void sdpa_bwd_short_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ lse,
    uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
    int H, int n, int m, float scale, float c_log2, int wl, int wr, int bottom_right,
    const int32_t* __restrict__ key_lens, const uint32_t* __restrict__ keep, float keep_scale) {
    constexpr int TB = tile_bytes<D>(), KS = D / 16, DT = D / 32, RB = D * 2;  // RB: bytes per row
    // [Q | dO | K | V] tiles, lse·log2 e and D of the 64 query rows, then (DROP)
    // the keep words.
    __shared__ __attribute__((aligned(1024))) char lds[4 * TB + 512 + (DROP ? 512 : 0)];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
    const int bh = blockIdx.x;
    const int b = bh / H;
    const size_t qbase = (size_t)bh * n * D, kvbase = (size_t)bh * m * D;
    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    // Each wave copies a quarter of the 1 KiB blocks of every tile.
    load_tile<D, 4>(lds, Q + qbase, 0, n, w, lane);
    load_tile<D, 4>(lds + TB, dO + qbase, 0, n, w, lane);
    load_tile<D, 4>(lds + 2 * TB, K + kvbase, 0, L, w, lane);
    load_tile<D, 4>(lds + 3 * TB, V + kvbase, 0, L, w, lane);
    const KeyWindow win{wl, wr, bottom_right ? L - n : 0, L};
    float* sl = reinterpret_cast<float*>(lds + 4 * TB);
    float* sdd = sl + 64;
    uint32_t* skw = reinterpret_cast<uint32_t*>(lds + 4 * TB + 512);  // DROP: [word][query]
    if constexpr (DROP) {
        // word w2 of query row q (zero past n and past the row's words)
        if (tid < 128) {
            const int q = tid & 63, w2 = tid >> 6, kwords = (m + 31) >> 5;
            skw[tid] = q < n && w2 < kwords ? keep[((size_t)bh * n + q) * kwords + w2] : 0u;
        }
    }

    TileAddr<D> ta;
    ta.init(lane);
    const uint32_t l0 = lds_u32(lds);
    const uint32_t sq = l0, sdo = l0 + TB, sk = l0 + 2 * TB, sv = l0 + 3 * TB;

    // dQ role: D and lse·log2 e of this wave's queries, from global O and dO.
    const int qrow = 32 * (w - 2) + l32;
    const bool qok = w >= 2 && qrow < n;
    float dsum = 0.f, lc = 0.f;
    if (w >= 2) {
        bf16x8 oop[KS], dop[KS];
        load_row_operand<D>(O + qbase + (size_t)qrow * D, qok, hf, oop);
        load_row_operand<D>(dO + qbase + (size_t)qrow * D, qok, hf, dop);
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)dop[ks][e], (float)oop[ks][e], acc);
        dsum = half_swap_sum(acc);
        const float lr = qok ? lse[(size_t)bh * n + qrow] : 0.f;
        lc = lr == -INFINITY ? INFINITY : lr * LOG2E;
        if (hf == 0) {
            sl[qrow] = lc;
            sdd[qrow] = dsum;
        }
    }
    wait_vmem();
    __syncthreads();

    f32x16 acc_a[DT], acc_b[DT];  // dQᵀ (waves 2, 3), or dKᵀ and dVᵀ (waves 0, 1)
    if (w >= 2) {
        // Sᵀ = K Qᵀ, dPᵀ = V dOᵀ over the 64 keys; dQᵀ += Kᵀ dSᵀ.
        bf16x8 qop[KS], dop[KS];
        {
            u32x4 r[2 * KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                r[ks] = ds_read_b128(sq + ta.row[ks] + (w - 2) * 32 * RB);
                r[KS + ks] = ds_read_b128(sdo + ta.row[ks] + (w - 2) * 32 * RB);
            }
            lds_wait(r);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qop[ks] = __builtin_bit_cast(bf16x8, r[ks]);
                dop[ks] = __builtin_bit_cast(bf16x8, r[KS + ks]);
            }
        }
        // Dropout: this query's keep words of keys 0..31 and 32..63.
        uint32_t kw[2] = {0u, 0u};
        if constexpr (DROP) {
            kw[0] = skw[qrow];
            kw[1] = skw[64 + qrow];
        }
        f32x16 s[2], dp[2];
        row_products<D, true>(sk, sv, ta, qop, dop, s, dp);
        const int llo = win.lo32(qrow) - 4 * hf, lhi = win.hi32(qrow) - 4 * hf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 32 * kt + 8 * (i >> 2) + (i & 3);
                const float sv_ = (off >= llo && off < lhi) ? s[kt][i] : -INFINITY;
                const float p = exp2_hw(__builtin_fmaf(sv_, c_log2, -lc));
                float g = dp[kt][i];
                if constexpr (DROP) g = (kw[kt] >> (8 * (i >> 2) + 4 * hf + (i & 3))) & 1u ? g * keep_scale : 0.f;
                s[kt][i] = p * (g - dsum);  // dSᵀ
            }
        bf16x8 db[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) db[j] = pack_step(s, j);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc_a[dt][i] = 0.f;
        tr_product<D>(sk, ta, db, acc_a);  // dQᵀ
    } else {
        // S = Q Kᵀ, dP = dO Vᵀ over the 64 queries; dVᵀ += dOᵀ P, dKᵀ += Qᵀ dS.
        const int key = 32 * w + l32;
        bf16x8 kop[KS], vop[KS];
        {
            u32x4 r[2 * KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                r[ks] = ds_read_b128(sk + ta.row[ks] + w * 32 * RB);
                r[KS + ks] = ds_read_b128(sv + ta.row[ks] + w * 32 * RB);
            }
            lds_wait(r);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kop[ks] = __builtin_bit_cast(bf16x8, r[ks]);
                vop[ks] = __builtin_bit_cast(bf16x8, r[KS + ks]);
            }
        }
        // Dropout: bit l32 of word w (this key's word) of every query row,
        // packed per 32-query half in the order of the S registers.
        uint32_t zb[2] = {0u, 0u};
        if constexpr (DROP) {
            u32x4 kv4[8];
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    kv4[4 * qh + gq] = ds_read_b128(lds_u32(skw) + (uint32_t)(64 * w + 32 * qh + 8 * gq + 4 * hf) * 4u);
            lds_wait(kv4);
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
#pragma unroll
                    for (int e = 0; e < 4; ++e) zb[qh] |= ((kv4[4 * qh + gq][e] >> l32) & 1u) << (4 * gq + e);
        }
        f32x16 s[2], dp[2];
        row_products<D, true>(sq, sdo, ta, kop, vop, s, dp);
        const QueryRange qr{wl, wr, bottom_right ? L - n : 0, L, n};
        const int llo = qr.qa(key) - 4 * hf, lhi = qr.qb(key) - 4 * hf;
        // The weights (query 32·qh + 8·(i/4) + 4·hf + i%4, this key) and dS, from
        // each query's lse·log2 e and D.
        if constexpr (D == 32) {
            // One 32-query half at a time: this keeps the kernel within the
            // 128 registers of four waves per SIMD (16 heads of 32 are twice
            // the workgroups of 8 heads of 64).
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) {
                u32x4 lv[4], dv4[4];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const uint32_t off = (uint32_t)(32 * qh + 8 * gq + 4 * hf) * 4u;
                    lv[gq] = ds_read_b128(l0 + 4 * TB + off);
                    dv4[gq] = ds_read_b128(l0 + 4 * TB + 256 + off);
                }
                lds_wait(lv);
                lds_wait(dv4);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int off = 32 * qh + 8 * (i >> 2) + (i & 3);
                    const float sv_ = (off >= llo && off < lhi) ? s[qh][i] : -INFINITY;
                    const float lcq = __uint_as_float(lv[i >> 2][i & 3]);
                    const float dd = __uint_as_float(dv4[i >> 2][i & 3]);
                    const float p = exp2_hw(__builtin_fmaf(sv_, c_log2, -lcq));
                    float g = dp[qh][i], pd = p;
                    if constexpr (DROP) {
                        const bool z = (zb[qh] >> i) & 1u;
                        pd = z ? p * keep_scale : 0.f;
                        g = z ? g * keep_scale : 0.f;
                    }
                    s[qh][i] = pd;             // the weights of dV
                    dp[qh][i] = p * (g - dd);  // dS
                }
            }
        } else {
        u32x4 lv[8], dv4[8];
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const uint32_t off = (uint32_t)(32 * qh + 8 * gq + 4 * hf) * 4u;
                lv[4 * qh + gq] = ds_read_b128(l0 + 4 * TB + off);
                dv4[4 * qh + gq] = ds_read_b128(l0 + 4 * TB + 256 + off);
            }
        lds_wait(lv);
        lds_wait(dv4);
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 32 * qh + 8 * (i >> 2) + (i & 3);
                const float sv_ = (off >= llo && off < lhi) ? s[qh][i] : -INFINITY;
                const float lcq = __uint_as_float(lv[4 * qh + (i >> 2)][i & 3]);
                const float dd = __uint_as_float(dv4[4 * qh + (i >> 2)][i & 3]);
                const float p = exp2_hw(__builtin_fmaf(sv_, c_log2, -lcq));
                float g = dp[qh][i], pd = p;
                if constexpr (DROP) {
                    const bool z = (zb[qh] >> i) & 1u;
                    pd = z ? p * keep_scale : 0.f;
                    g = z ? g * keep_scale : 0.f;
                }
                s[qh][i] = pd;             // the weights of dV
                dp[qh][i] = p * (g - dd);  // dS
            }
        }
        bf16x8 pb[4], db[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pb[j] = pack_step(s, j);
            db[j] = pack_step(dp, j);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) { acc_a[dt][i] = 0.f; acc_b[dt][i] = 0.f; }
        tr_product<D>(sdo, ta, pb, acc_b);  // dVᵀ
        tr_product<D>(sq, ta, db, acc_a);   // dKᵀ
    }
    // Every wave is done with the tiles: their space now stages the outputs
    // in 64·D-byte areas (wave w < 2: dK at area 2·w, dV at 2·w + 1; waves 2,
    // 3: dQ at area 4 + w − 2).
    __syncthreads();
    constexpr int AREA = 32 * RB;
    if (w >= 2) {
        const int r0 = 32 * (w - 2);
        store_rows_lds<D>(lds + (2 + w) * AREA, acc_a, lane, scale, dQ + qbase + (size_t)r0 * D, n - r0);
    } else {
        const int r0 = 32 * w;
        store_rows_lds<D>(lds + 2 * w * AREA, acc_a, lane, scale, dK + kvbase + (size_t)r0 * D, m - r0);
        store_rows_lds<D>(lds + (2 * w + 1) * AREA, acc_b, lane, 1.f, dV + kvbase + (size_t)r0 * D, m - r0);
    }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int n) { return 2 * (((size_t)B * H * n * 4 + 255) & ~(size_t)255); }

namespace {

template <int D, int NW, bool DROP>
hipError_t launch_bwd_width(const BwdArgs& a, hipStream_t stream, float c_log2, float* ws_d, float* ws_l) {
    const int BH = a.B * a.H;
    const int nqb = (a.n + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((sdpa_bwd_dq_bf16<D, NW, DROP>), dim3(nqb * BH), dim3(NW * 64), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.out, (const uint16_t*)a.dout, a.lse, (uint16_t*)a.dq,
                       ws_d, ws_l, BH, a.H, a.n, a.m, a.scale, c_log2, a.wl, a.wr, a.bottom_right,
                       a.key_lens, nqb, a.keep, a.keep_scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid(((a.m + 32 * NW - 1) / (32 * NW)) * BH);
    // Both gradients in one launch for D <= 64; at D = 128 one launch each
    // keeps the accumulators within the register file.
    constexpr bool ONE = D <= 64;
    hipLaunchKernelGGL((sdpa_bwd_dkdv_bf16<D, NW, true, ONE, DROP>), grid, dim3(NW * 64), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, ws_d, ws_l, (uint16_t*)a.dk, (uint16_t*)a.dv, BH, a.H,
                       a.n, a.m, a.scale, c_log2, a.wl, a.wr, a.bottom_right, a.key_lens, a.keep,
                       a.keep_scale);
    if constexpr (!ONE) {
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((sdpa_bwd_dkdv_bf16<D, NW, false, true, DROP>), grid, dim3(NW * 64), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, ws_d, ws_l, (uint16_t*)a.dk, (uint16_t*)a.dv, BH, a.H,
                           a.n, a.m, a.scale, c_log2, a.wl, a.wr, a.bottom_right, a.key_lens, a.keep,
                           a.keep_scale);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream, float c_log2, float* ws_d, float* ws_l) {
    // 4 waves per workgroup once there are enough query blocks to fill the chip.
    const bool four = (long long)a.B * a.H * ((a.n + 127) / 128) >= 1024;
    if (a.keep)
        return four ? launch_bwd_width<D, 4, true>(a, stream, c_log2, ws_d, ws_l)
                    : launch_bwd_width<D, 2, true>(a, stream, c_log2, ws_d, ws_l);
    return four ? launch_bwd_width<D, 4, false>(a, stream, c_log2, ws_d, ws_l)
                : launch_bwd_width<D, 2, false>(a, stream, c_log2, ws_d, ws_l);
}

template <int D>
hipError_t launch_bwd_short(const BwdArgs& a, hipStream_t stream, float c_log2) {
    const auto kernel = a.keep ? sdpa_bwd_short_bf16<D, true> : sdpa_bwd_short_bf16<D, false>;
    hipLaunchKernelGGL(kernel, dim3(a.B * a.H), dim3(256), 0, stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.out,
                       (const uint16_t*)a.dout, a.lse, (uint16_t*)a.dq, (uint16_t*)a.dk, (uint16_t*)a.dv,
                       a.H, a.n, a.m, a.scale, c_log2, a.wl, a.wr, a.bottom_right, a.key_lens, a.keep,
                       a.keep_scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    float* ws_d = static_cast<float*>(a.workspace);
    float* ws_l = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + bwd_workspace_bytes(a.B, a.H, a.n) / 2);
    if (a.n <= 64 && a.m <= 64) {
        if (a.d == 32) return launch_bwd_short<32>(a, stream, c_log2);
        if (a.d == 128) return launch_bwd_short<128>(a, stream, c_log2);
        return launch_bwd_short<64>(a, stream, c_log2);
    }
    if (a.d == 32) return launch_bwd_d<32>(a, stream, c_log2, ws_d, ws_l);
    if (a.d == 128) return launch_bwd_d<128>(a, stream, c_log2, ws_d, ws_l);
    return launch_bwd_d<64>(a, stream, c_log2, ws_d, ws_l);
}

}  // namespace sdpa
