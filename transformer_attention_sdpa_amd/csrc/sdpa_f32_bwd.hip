// Gradient of scaled dot-product attention for fp32 inputs on gfx950, at
// head width d_k = d_v = 64.
//
// Eq. (1) of 《精读 Attention Is All You Need：原始 Transformer 论文》 is the
// forward pass; the pages train through it in single precision.  By the chain
// rule, with s = scale·q·k, P = softmax(S) row-wise and O = P V:
//
//   dV = Pᵀ dO,   dP = dO Vᵀ,   dS = P ∘ (dP − D),   D_i = dO_i · O_i,
//   dQ = scale · dS K,   dK = scale · dSᵀ Q.
//
// P is recomputed tile by tile from the forward pass's per-row log-sum-exp,
// P_ij = 2^(s_ij·log2 e − lse_i·log2 e).  fp32 end to end: every product on
// v_mfma_f32_32x32x2_f32 (full fp32 operands; gfx950 has no truncated xf32
// form), fp32 weights, fp32 gradients.  Two launches, no atomics, so the
// result is bitwise reproducible:
//
//   1. sdpa_bwd_dq_f32, one wave per 32 queries: writes D_i and lse_i·log2 e
//      of its rows to the workspace, then streams the K/V tiles its queries
//      may see:  Sᵀ = K Qᵀ, dPᵀ = V dOᵀ, dSᵀ = Pᵀ ∘ (dPᵀ − D), dQᵀ += Kᵀ dSᵀ.
//   2. sdpa_bwd_dkdv_f32, one wave per 32 keys: streams the Q/dO tiles (and
//      their D and lse values) of the queries that may see its keys:
//      S = Q Kᵀ, dP = dO Vᵀ, dS = P ∘ (dP − D), dVᵀ += dOᵀ P, dKᵀ += Qᵀ dS.
//
// Layout of the products (as in the fp32 forward kernel): a lane holds one
// column of each 32×32 result — the query (launch 1) or the key (launch 2) it
// owns — and rows 8·(i/4) + 4·hf + i%4 in register i (hf = lane / 32).  The
// first two products contract over d with A read from LDS rows and B held in
// VGPRs; in the last ones that register layout is the B operand as it stands
// (step i contracts row 8·(i/4) + 4·hf + i%4 for half-wave hf), and A is one
// float per lane read from the row-major tile, so no transpose is needed.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int D = kHeadDim;  // 64
constexpr int BT = 32;       // rows per LDS tile (keys in launch 1, queries in launch 2)
constexpr float LOG2E = 1.4426950408889634f;

// 16-byte chunk c (0..15) of tile row r sits at chunk position c ^ (r & 15).
__device__ __forceinline__ int swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

// Element (r, col) of a swizzled tile as a float index.
__device__ __forceinline__ int swz_elem(int r, int col) { return swz(r, col >> 2) * 4 + (col & 3); }

// This lane's half of a 64-float row as the B operand of a d-contraction:
// floats 32·hf .. 32·hf + 31 (zeros if !ok).
__device__ __forceinline__ void load_half_row(const float* row, bool ok, int hf, float (&x)[32]) {
    if (ok) {
        const f32x4* src = reinterpret_cast<const f32x4*>(row + 32 * hf);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const f32x4 v = src[c];
            x[4 * c + 0] = v[0]; x[4 * c + 1] = v[1]; x[4 * c + 2] = v[2]; x[4 * c + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = 0.f;
    }
}

// acc (32 tile rows × this lane's column) += tile · b over d: step (c, e)
// contracts d = 4c + e (half-wave 0) and 32 + 4c + e (half-wave 1).
__device__ __forceinline__ void row_product(const f32x4* tile, int l32, int hf, const float (&b)[32],
                                            f32x16& acc) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const f32x4 a4 = tile[swz(l32, 8 * hf + c)];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma32x32x2_f32(a4[e], b[4 * c + e], acc);
    }
}

// acc[dt] (dims 32·dt + rows × this lane's column) += tileᵀ · x, contracting
// the tile's 32 rows in the order of x's registers.
__device__ __forceinline__ void col_product(const float* tile, int l32, int hf, const f32x16& x,
                                            f32x16 (&acc)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * hf + (i & 3);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) acc[dt] = mfma32x32x2_f32(tile[swz_elem(r, 32 * dt + l32)], x[i], acc[dt]);
    }
}

// Row `row` of a [.., 64] fp32 tensor from an accumulator pair (dims 32·dt +
// 8·(i/4) + 4·hf + i%4 in register i of acc[dt]), times f: 16-byte stores.
__device__ __forceinline__ void store_row(float* row, const f32x16 (&acc)[2], int hf, float f) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 o;
            o[0] = acc[dt][4 * i4 + 0] * f;
            o[1] = acc[dt][4 * i4 + 1] * f;
            o[2] = acc[dt][4 * i4 + 2] * f;
            o[3] = acc[dt][4 * i4 + 3] * f;
            *reinterpret_cast<f32x4*>(row + 32 * dt + 8 * i4 + 4 * hf) = o;
        }
}

// Register staging of one pair of 32-row tiles (rows at or past `rows` are
// zeros): global → VGPRs during the previous tile's math, then VGPRs → LDS.
template <int NT>
struct TilePair {
    static constexpr int CHUNKS = BT * D / 4;  // 512 16-byte chunks per tile
    static constexpr int CPT = (CHUNKS + NT - 1) / NT;
    f32x4 ra[CPT], rb[CPT];
    __device__ __forceinline__ void load(const float* A, const float* Bt, int r0, int rows, int tid) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            const int r = r0 + (c >> 4);
            if (c < CHUNKS && r < rows) {
                ra[i] = reinterpret_cast<const f32x4*>(A + (size_t)r * D)[c & 15];
                rb[i] = reinterpret_cast<const f32x4*>(Bt + (size_t)r * D)[c & 15];
            } else {
                ra[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                rb[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    __device__ __forceinline__ void store(f32x4* sa, f32x4* sb, int tid) const {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            if (c < CHUNKS) {
                sa[swz(c >> 4, c & 15)] = ra[i];
                sb[swz(c >> 4, c & 15)] = rb[i];
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Launch 1: dQ, and D and lse·log2 e of every query row for launch 2.
template <int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_bwd_dq_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ dQ, float* __restrict__ ws_d, float* __restrict__ ws_l, int BH, int H, int n,
    int m, float scale, float c_log2, int wl, int wr, int bottom_right, const int32_t* __restrict__ key_lens,
    int nqb) {
    constexpr int NT = NW * 64;
    __shared__ f32x4 sK[BT * 16];
    __shared__ f32x4 sV[BT * 16];
    const int tid = threadIdx.x;
    const int w = tid >> 6;
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
    const int kbeg = win.lo(q0), kend = win.hi(min(q0 + 32 * NW, n) - 1);
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
    const int qlo = win.lo(qrow), qhi = win.hi(qrow);
    float qop[32], dop[32];
    load_half_row(Q + qbase + (size_t)qrow * D, qok, hf, qop);
    load_half_row(dO + qbase + (size_t)qrow * D, qok, hf, dop);
    // D_i = dO_i · O_i over this lane's half of the dims, then the other half-wave's.
    float dsum;
    {
        float oop[32];
        load_half_row(O + qbase + (size_t)qrow * D, qok, hf, oop);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc = __builtin_fmaf(dop[e], oop[e], acc);
        dsum = half_swap_sum(acc);
    }
    // P = 2^(s·c − lc); a row with no legal key (lse = −∞) gets lc = +∞, P = 0.
    const float lr = qok ? lse[(size_t)bh * n + qrow] : 0.f;
    const float lc = lr == -INFINITY ? INFINITY : lr * LOG2E;
    if (qok && hf == 0) {
        ws_d[(size_t)bh * n + qrow] = dsum;
        ws_l[(size_t)bh * n + qrow] = lc;
    }

    f32x16 acc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][i] = acc[1][i] = 0.f;
    const float* sKf = reinterpret_cast<const float*>(sK);
    TilePair<NT> st;
    if (tend > tbeg) st.load(K + kvbase, V + kvbase, tbeg * BT, L, tid);
    for (int t = tbeg; t < tend; ++t) {
        __syncthreads();
        st.store(sK, sV, tid);
        __syncthreads();
        if (t + 1 < tend) st.load(K + kvbase, V + kvbase, (t + 1) * BT, L, tid);

        const int k0 = t * BT;
        if (k0 >= whi || k0 + BT <= wlo) continue;  // no query of this wave sees the tile

        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
        row_product(sK, l32, hf, qop, s);   // Sᵀ = K Qᵀ
        row_product(sV, l32, hf, dop, dp);  // dPᵀ = V dOᵀ
        // Register i is key k0 + 8·(i/4) + 4·hf + i%4 of query qrow.
        if (k0 < flo || k0 + BT > fhi) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + 8 * (i >> 2) + 4 * hf + (i & 3);
                if (key < qlo || key >= qhi) s[i] = -INFINITY;
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = exp2_hw(__builtin_fmaf(s[i], c_log2, -lc));
            s[i] = p * (dp[i] - dsum);  // dSᵀ
        }
        col_product(sKf, l32, hf, s, acc);  // dQᵀ += Kᵀ dSᵀ
    }
    if (qok) store_row(dQ + qbase + (size_t)qrow * D, acc, hf, scale);
}

// ---------------------------------------------------------------------------
// Launch 2: dK, dV.

// Queries that may see key j form the interval [qa, qb) (the legal keys of a
// query, [lo_i, hi_i), move right with i).  Keys at or past L see none.
struct QueryInterval {
    int wl, wr, shift, L, n;
    __device__ __forceinline__ int qa(int j) const {
        if (j >= L || wr < 0) return 0;
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

template <int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_bwd_dkdv_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ ws_d, const float* __restrict__ ws_l,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int H, int n, int m, float scale,
    float c_log2, int wl, int wr, int bottom_right, const int32_t* __restrict__ key_lens) {
    constexpr int NT = NW * 64;
    __shared__ f32x4 sQ[BT * 16];
    __shared__ f32x4 sG[BT * 16];  // the dO tile
    __shared__ f32x4 sL[BT / 4];   // lse·log2 e of the tile's queries
    __shared__ f32x4 sDs[BT / 4];  // D of the tile's queries
    const int tid = threadIdx.x;
    const int w = tid >> 6;
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
    const QueryInterval qr{wl, wr, bottom_right ? L - n : 0, L, n};
    // Queries [qbeg, qend) see some key of the block.
    const int klast = min(k0 + 32 * NW, L) - 1;
    const int qbeg = klast >= k0 ? qr.qa(k0) : 0;
    const int qend = klast >= k0 ? qr.qb(klast) : 0;
    const int tbeg = qbeg / BT;
    const int tend = qend > qbeg ? (qend + BT - 1) / BT : tbeg;
    // This wave's keys: queries [wqa, wqb) needed, [fqa, fqb) see all of them
    // (a wave holding keys past L never has a tile legal for all of them).
    const int wk0 = k0 + 32 * w;
    const int wlast = min(wk0 + 32, L) - 1;
    const bool wact = wlast >= wk0;
    const int wqa = wact ? qr.qa(wk0) : 0, wqb = wact ? qr.qb(wlast) : 0;
    const bool wfull = wact && wk0 + 31 < L;
    const int fqa = wfull ? qr.qa(wlast) : 0, fqb = wfull ? qr.qb(wk0) : 0;

    const size_t qbase = (size_t)bh * n * D, kvbase = (size_t)bh * m * D;
    const int key = wk0 + l32;
    // Kᵀ, Vᵀ as B operands; keys at or past L are zeros (their rows may hold
    // anything), so their logits are masked and their gradients are exactly 0.
    float kop[32], vop[32];
    load_half_row(K + kvbase + (size_t)key * D, key < L, hf, kop);
    load_half_row(V + kvbase + (size_t)key * D, key < L, hf, vop);
    const int ka = qr.qa(key), kb = qr.qb(key);

    f32x16 dka[2], dva[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[0][i] = dka[1][i] = dva[0][i] = dva[1][i] = 0.f;
    const float* sQf = reinterpret_cast<const float*>(sQ);
    const float* sGf = reinterpret_cast<const float*>(sG);
    TilePair<NT> st;
    float rl = 0.f, rd = 0.f;  // lse·log2 e and D of query row t·BT + tid (tid < BT)
    auto load_rows = [&](int t) {
        const int r = t * BT + tid;
        rl = tid < BT && r < n ? ws_l[(size_t)bh * n + r] : 0.f;
        rd = tid < BT && r < n ? ws_d[(size_t)bh * n + r] : 0.f;
    };
    if (tend > tbeg) {
        st.load(Q + qbase, dO + qbase, tbeg * BT, n, tid);
        load_rows(tbeg);
    }
    for (int t = tbeg; t < tend; ++t) {
        __syncthreads();
        st.store(sQ, sG, tid);
        if (tid < BT) {
            reinterpret_cast<float*>(sL)[tid] = rl;
            reinterpret_cast<float*>(sDs)[tid] = rd;
        }
        __syncthreads();
        if (t + 1 < tend) {
            st.load(Q + qbase, dO + qbase, (t + 1) * BT, n, tid);
            load_rows(t + 1);
        }

        const int t0 = t * BT;
        if (t0 >= wqb || t0 + BT <= wqa) continue;  // no query of the tile sees a key of the wave

        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
        row_product(sQ, l32, hf, kop, s);   // S = Q Kᵀ
        row_product(sG, l32, hf, vop, dp);  // dP = dO Vᵀ
        // Register i is query t0 + 8·(i/4) + 4·hf + i%4 of key `key`.
        if (t0 < fqa || t0 + BT > fqb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = t0 + 8 * (i >> 2) + 4 * hf + (i & 3);
                if (q < ka || q >= kb) s[i] = -INFINITY;
            }
        }
        // Those queries' lse·log2 e and D: four consecutive floats per group
        // of four registers.
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 lc = sL[2 * i4 + hf];
            const f32x4 dd = sDs[2 * i4 + hf];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * i4 + e;
                const float p = exp2_hw(__builtin_fmaf(s[i], c_log2, -lc[e]));
                s[i] = p;
                dp[i] = p * (dp[i] - dd[e]);  // dS
            }
        }
        col_product(sGf, l32, hf, s, dva);   // dVᵀ += dOᵀ P
        col_product(sQf, l32, hf, dp, dka);  // dKᵀ += Qᵀ dS
    }
    if (key < m) {
        store_row(dK + kvbase + (size_t)key * D, dka, hf, scale);
        store_row(dV + kvbase + (size_t)key * D, dva, hf, 1.f);
    }
}

// ---------------------------------------------------------------------------
// Split forms, for grids too small to fill the chip with one wave per 32 rows
// (sentence-length batches): a workgroup owns one block of 32 queries (dQ) or
// keys (dK, dV), and its NW waves take every NW-th tile of the stream (wave w:
// tiles tbeg + w, tbeg + w + NW, …), each into tiles of its own in LDS
// (buffer_load … lds, no barrier between waves).  The partial gradients are
// then summed through LDS in wave order, so the result stays deterministic.

// Rows [r0, r0 + 32) of a [rows, 64] fp32 tensor (rows past `rows` read as
// zeros) into a swizzled 8 KiB LDS tile, by this wave alone: load u fills rows
// 4u .. 4u + 3; lane ln lands at (row 4u + ln / 16, position ln % 16), which
// holds chunk (ln % 16) ^ (row mod 16).
__device__ __forceinline__ void wave_tile_load(const float* base, int rows, int r0, f32x4* tile, int lane) {
    const i32x4 rs = make_rsrc(base, rows > 0 ? (uint32_t)rows * (uint32_t)(D * 4) : 0u);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int row = 4 * u + (lane >> 4);
        const int c = (lane & 15) ^ (row & 15);
        load16_to_lds(rs, tile + 64 * u, (r0 + row) * D * 4 + c * 16);
    }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_bwd_dq_f32_split(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ O, const float* __restrict__ dO, const float* __restrict__ lse,
    float* __restrict__ dQ, float* __restrict__ ws_d, float* __restrict__ ws_l, int BH, int H, int n,
    int m, float scale, float c_log2, int wl, int wr, int bottom_right, const int32_t* __restrict__ key_lens,
    int nqb) {
    __shared__ f32x4 lds[NW][2][BT * 16];  // per wave: K tile, V tile
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;

    const int g = blockIdx.x;
    const int bh = g % BH;
    const int q0 = (nqb - 1 - g / BH) * 32;
    const int b = bh / H;
    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    const KeyWindow win{wl, wr, bottom_right ? L - n : 0, L};
    const int qlast = min(q0 + 32, n) - 1;
    const int kbeg = win.lo(q0), kend = win.hi(qlast);
    const int tbeg = kbeg / BT;
    const int tend = kend > kbeg ? (kend + BT - 1) / BT : tbeg;
    const int flo = win.lo(qlast), fhi = win.hi(q0);  // keys legal for every query of the block

    const size_t qbase = (size_t)bh * n * D, kvbase = (size_t)bh * m * D;
    f32x4* sK = lds[w][0];
    f32x4* sV = lds[w][1];
    // The first tile is requested before the row operands, so that both
    // round trips to memory overlap.
    if (tbeg + w < tend) {
        wave_tile_load(K + kvbase, L, (tbeg + w) * BT, sK, lane);
        wave_tile_load(V + kvbase, L, (tbeg + w) * BT, sV, lane);
    }
    const int qrow = q0 + l32;
    const bool qok = qrow < n;
    const int qlo = win.lo(qrow), qhi = win.hi(qrow);
    float qop[32], dop[32];
    load_half_row(Q + qbase + (size_t)qrow * D, qok, hf, qop);
    load_half_row(dO + qbase + (size_t)qrow * D, qok, hf, dop);
    float dsum;
    {
        float oop[32];
        load_half_row(O + qbase + (size_t)qrow * D, qok, hf, oop);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc = __builtin_fmaf(dop[e], oop[e], acc);
        dsum = half_swap_sum(acc);
    }
    const float lr = qok ? lse[(size_t)bh * n + qrow] : 0.f;
    const float lc = lr == -INFINITY ? INFINITY : lr * LOG2E;
    if (w == 0 && qok && hf == 0) {
        ws_d[(size_t)bh * n + qrow] = dsum;
        ws_l[(size_t)bh * n + qrow] = lc;
    }

    f32x16 acc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][i] = acc[1][i] = 0.f;
    for (int t = tbeg + w; t < tend; t += NW) {
        if (t != tbeg + w) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the previous tile's reads are done
            wave_tile_load(K + kvbase, L, t * BT, sK, lane);
            wave_tile_load(V + kvbase, L, t * BT, sV, lane);
        }
        wait_vmem();
        const int k0 = t * BT;
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
        row_product(sK, l32, hf, qop, s);   // Sᵀ = K Qᵀ
        row_product(sV, l32, hf, dop, dp);  // dPᵀ = V dOᵀ
        if (k0 < flo || k0 + BT > fhi) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + 8 * (i >> 2) + 4 * hf + (i & 3);
                if (key < qlo || key >= qhi) s[i] = -INFINITY;
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = exp2_hw(__builtin_fmaf(s[i], c_log2, -lc));
            s[i] = p * (dp[i] - dsum);  // dSᵀ
        }
        col_product(reinterpret_cast<const float*>(sK), l32, hf, s, acc);  // dQᵀ += Kᵀ dSᵀ
    }

    // dQ = Σ_w partial_w in wave order: waves 1.. park theirs in LDS.
    __syncthreads();
    float* red = reinterpret_cast<float*>(&lds[0][0][0]);
    if (w > 0) {
#pragma unroll
        for (int r = 0; r < 32; ++r) red[((w - 1) * 32 + r) * 64 + lane] = acc[r >> 4][r & 15];
    }
    __syncthreads();
    if (w == 0 && qok) {
#pragma unroll
        for (int u = 1; u < NW; ++u)
#pragma unroll
            for (int r = 0; r < 32; ++r) acc[r >> 4][r & 15] += red[((u - 1) * 32 + r) * 64 + lane];
        store_row(dQ + qbase + (size_t)qrow * D, acc, hf, scale);
    }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_bwd_dkdv_f32_split(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ ws_d, const float* __restrict__ ws_l,
    float* __restrict__ dK, float* __restrict__ dV, int BH, int H, int n, int m, float scale,
    float c_log2, int wl, int wr, int bottom_right, const int32_t* __restrict__ key_lens) {
    // per wave: Q tile, dO tile, then lse·log2 e and D of the tile's rows
    // (64 floats each: the 4-byte loads fill a whole wave's worth)
    __shared__ f32x4 lds[NW][2 * BT * 16 + 32];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hf = lane >> 5;

    const int g = blockIdx.x;
    const int bh = g % BH;
    const int k0 = (g / BH) * 32;
    const int b = bh / H;
    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    const QueryInterval qr{wl, wr, bottom_right ? L - n : 0, L, n};
    const int klast = min(k0 + 32, L) - 1;
    const bool any = klast >= k0;
    const int qbeg = any ? qr.qa(k0) : 0;
    const int qend = any ? qr.qb(klast) : 0;
    const int tbeg = qbeg / BT;
    const int tend = qend > qbeg ? (qend + BT - 1) / BT : tbeg;
    const bool full = any && k0 + 31 < L;
    const int fqa = full ? qr.qa(klast) : 0, fqb = full ? qr.qb(k0) : 0;

    const size_t qbase = (size_t)bh * n * D, kvbase = (size_t)bh * m * D;
    f32x4* sQ = lds[w];
    f32x4* sG = lds[w] + BT * 16;
    f32x4* sL = lds[w] + 2 * BT * 16;       // 64 floats
    f32x4* sDs = lds[w] + 2 * BT * 16 + 16; // 64 floats
    auto issue = [&](int t0) {
        wave_tile_load(Q + qbase, n, t0, sQ, lane);
        wave_tile_load(dO + qbase, n, t0, sG, lane);
        const uint32_t nb = (uint32_t)max(n - t0, 0) * 4u;  // rows past n read as zeros
        sdpa_llvm_buffer_load_lds(make_rsrc(ws_l + (size_t)bh * n + t0, nb),
                                  (__attribute__((address_space(3))) void*)sL, 4, lane * 4, 0, 0, 0);
        sdpa_llvm_buffer_load_lds(make_rsrc(ws_d + (size_t)bh * n + t0, nb),
                                  (__attribute__((address_space(3))) void*)sDs, 4, lane * 4, 0, 0, 0);
    };
    // The first tile is requested before the row operands (both round trips overlap).
    if (tbeg + w < tend) issue((tbeg + w) * BT);
    const int key = k0 + l32;
    float kop[32], vop[32];
    load_half_row(K + kvbase + (size_t)key * D, key < L, hf, kop);
    load_half_row(V + kvbase + (size_t)key * D, key < L, hf, vop);
    const int ka = qr.qa(key), kb = qr.qb(key);

    f32x16 dka[2], dva[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[0][i] = dka[1][i] = dva[0][i] = dva[1][i] = 0.f;
    for (int t = tbeg + w; t < tend; t += NW) {
        const int t0 = t * BT;
        if (t != tbeg + w) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the previous tile's reads are done
            issue(t0);
        }
        wait_vmem();
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
        row_product(sQ, l32, hf, kop, s);   // S = Q Kᵀ
        row_product(sG, l32, hf, vop, dp);  // dP = dO Vᵀ
        if (t0 < fqa || t0 + BT > fqb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int q = t0 + 8 * (i >> 2) + 4 * hf + (i & 3);
                if (q < ka || q >= kb) s[i] = -INFINITY;
            }
        }
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 lc = sL[2 * i4 + hf];
            const f32x4 dd = sDs[2 * i4 + hf];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * i4 + e;
                const float p = exp2_hw(__builtin_fmaf(s[i], c_log2, -lc[e]));
                s[i] = p;
                dp[i] = p * (dp[i] - dd[e]);  // dS
            }
        }
        col_product(reinterpret_cast<const float*>(sG), l32, hf, s, dva);   // dVᵀ += dOᵀ P
        col_product(reinterpret_cast<const float*>(sQ), l32, hf, dp, dka);  // dKᵀ += Qᵀ dS
    }

    // dK, dV = Σ_w partial_w in wave order: waves 1.. park theirs in LDS.
    __syncthreads();
    float* red = reinterpret_cast<float*>(&lds[0][0]);
    if (w > 0) {
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            red[((w - 1) * 64 + r) * 64 + lane] = dka[r >> 4][r & 15];
            red[((w - 1) * 64 + 32 + r) * 64 + lane] = dva[r >> 4][r & 15];
        }
    }
    __syncthreads();
    if (w == 0 && key < m) {
#pragma unroll
        for (int u = 1; u < NW; ++u)
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                dka[r >> 4][r & 15] += red[((u - 1) * 64 + r) * 64 + lane];
                dva[r >> 4][r & 15] += red[((u - 1) * 64 + 32 + r) * 64 + lane];
            }
        store_row(dK + kvbase + (size_t)key * D, dka, hf, scale);
        store_row(dV + kvbase + (size_t)key * D, dva, hf, 1.f);
    }
}

}  // namespace

namespace {

template <int NW>
hipError_t launch_dq_split(const BwdArgs& a, hipStream_t stream, float c_log2, float* ws_d, float* ws_l) {
    const int BH = a.B * a.H;
    const int nqb = (a.n + 31) / 32;
    hipLaunchKernelGGL(sdpa_bwd_dq_f32_split<NW>, dim3(nqb * BH), dim3(NW * 64), 0, stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.out, (const float*)a.dout, a.lse,
                       (float*)a.dq, ws_d, ws_l, BH, a.H, a.n, a.m, a.scale, c_log2, a.wl, a.wr, a.bottom_right,
                       a.key_lens, nqb);
    return hipGetLastError();
}

template <int NW>
hipError_t launch_dkdv_split(const BwdArgs& a, hipStream_t stream, float c_log2, float* ws_d, float* ws_l) {
    const int BH = a.B * a.H;
    hipLaunchKernelGGL(sdpa_bwd_dkdv_f32_split<NW>, dim3(((a.m + 31) / 32) * BH), dim3(NW * 64), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout, ws_d, ws_l,
                       (float*)a.dk, (float*)a.dv, BH, a.H, a.n, a.m, a.scale, c_log2, a.wl, a.wr,
                       a.bottom_right, a.key_lens);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t stream) {
    constexpr int NW = 2;
    const int BH = a.B * a.H;
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    float* ws_d = static_cast<float*>(a.workspace);
    float* ws_l = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + bwd_workspace_bytes(a.B, a.H, a.n) / 2);
    // Fewer than 1024 blocks of 64 rows (four waves per CU): the split forms.
    // Each launch's waves split the tiles it streams: four once there are
    // more than three (dQ streams keys, dK/dV queries).
    if ((long long)BH * ((a.n + 63) / 64) < 1024 && (long long)BH * ((a.m + 63) / 64) < 1024) {
        const hipError_t e = a.m > 96 ? launch_dq_split<4>(a, stream, c_log2, ws_d, ws_l)
                                      : launch_dq_split<2>(a, stream, c_log2, ws_d, ws_l);
        if (e != hipSuccess) return e;
        return a.n > 96 ? launch_dkdv_split<4>(a, stream, c_log2, ws_d, ws_l)
                        : launch_dkdv_split<2>(a, stream, c_log2, ws_d, ws_l);
    }
    const int nqb = (a.n + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL(sdpa_bwd_dq_f32<NW>, dim3(nqb * BH), dim3(NW * 64), 0, stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.out, (const float*)a.dout, a.lse,
                       (float*)a.dq, ws_d, ws_l, BH, a.H, a.n, a.m, a.scale, c_log2, a.wl, a.wr, a.bottom_right,
                       a.key_lens, nqb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nkb = (a.m + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL(sdpa_bwd_dkdv_f32<NW>, dim3(nkb * BH), dim3(NW * 64), 0, stream, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (const float*)a.dout, ws_d, ws_l, (float*)a.dk,
                       (float*)a.dv, BH, a.H, a.n, a.m, a.scale, c_log2, a.wl, a.wr, a.bottom_right, a.key_lens);
    return hipGetLastError();
}

}  // namespace sdpa
