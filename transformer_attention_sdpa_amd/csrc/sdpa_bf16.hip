// Fused single-pass attention forward for bf16 inputs on gfx950 (MI355X),
// for any n and m (the long-sequence path; n, m <= 64 take the short kernel).
//
// Computes Eq. (1) of 《精读 Attention Is All You Need：原始 Transformer 论文》
// ("缩放点积注意力：点积为什么要缩放"), softmax(Q Kᵀ·scale) V, for every
// (batch, head) pair, with the decoder's illegal logits set to −∞ before the
// softmax (《Attention Is All You Need：注意力就是你所需要的一切》 §3.2.3) and key
// padding handled the same way.  The mask is a key window around each query
// (KeyWindow): the causal mask, and the restricted attention of the same
// pages' Table 1, are both windows.  Scores and softmax are fp32; the weights are
// rounded to bf16 (RNE) for the P·V product, which accumulates in fp32; the
// output is rounded once to bf16.
//
// Work layout.  A workgroup owns BM = NW·64 consecutive queries of one head;
// each wave owns 64 of them as two 32-query sub-blocks (QT = 2) that share
// every K/V operand read from LDS.  Keys stream through LDS in tiles of 64 rows
// (K and V, 8 KiB each), double-buffered, one barrier per tile.  Tiles move
// HBM → LDS with buffer_load_dwordx4 … lds (no VGPR staging); the buffer range
// ends at the sequence's key length, so rows past it arrive as zeros without
// being read.  Each wave keeps a running reference maximum and sum per query
// (online softmax), so no n×m score matrix ever exists.  Both products run on
// v_mfma_f32_32x32x16_bf16, computed transposed:
//
//   Sᵀ (64 keys × 32 queries)  = K · Qᵀ          A = K rows from LDS, B = Qᵀ in VGPRs
//   Oᵀ (64 dv  × 32 queries) += Vᵀ · Pᵀ          A = Vᵀ via LDS transpose reads,
//                                                B = Pᵀ straight from the Sᵀ registers
//
// so every lane holds one query's column: the row max/sum are lane-local plus
// one exchange between half-waves, and the rescale of Oᵀ is a per-lane multiply.
//
// VALU economy (at d = 64 the softmax costs about as much issue time as the
// matrix products):
//   * the weights are formed against a reference maximum that only moves when a
//     tile's weights would exceed 2^14 (checked on the row sums, so the tile
//     maximum is not even computed on most tiles), and the Oᵀ/l rescale only
//     happens then — exact, because any common reference cancels in
//     Σ p·v / Σ p;
//   * one FMA + one v_exp_f32 per score (scale·log2 e folded into the FMA);
//   * row sums with v_dot2_f32_bf16 on the packed bf16 weights (the same values
//     that enter P·V);
//   * masking (selects to −∞) only on tiles that straddle a window edge (the
//     causal diagonal is one) or the padding edge; the tile loop covers only
//     the keys the workgroup's queries may see, and a wave skips tiles wholly
//     outside its own queries' windows;
//   * LDS addresses are per-lane constants plus immediate offsets (the tile
//     loop is unrolled by two so the buffer index is a constant).
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int D = kHeadDim;  // 64
constexpr int BN = 64;       // keys per LDS tile
constexpr int QT = 2;        // 32-query sub-blocks per wave
constexpr int QW = 32 * QT;  // queries per wave
// A lane's partial weight sum over one tile may reach this before the reference
// maximum moves: weights stay below it (2^14), far inside bf16 and fp32 range.
constexpr float SUM_LIMIT = 16384.f;
constexpr int TILE_BYTES = BN * D * 2;  // 8 KiB

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// STRIDED: K/V row strides from the caller's layout; else the packed D.
// DROP: attention dropout with a keep-bit mask (weights of dropped pairs leave
// the P·V product, not the row sums; the output is scaled by keep_scale).
template <int NW, bool STRIDED, bool DROP>
struct LongKernel {
    static constexpr int NT = NW * 64;
    static constexpr int BM = NW * QW;
    static constexpr int LOADS = TILE_BYTES / 1024 / NW;  // 1 KiB loads per wave per tensor per tile

    // LDS: [buf][K | V] tiles of 8 KiB; 16-byte chunk c of row r at lds_swz(r, c).
    char* lds;
    // Per-lane constants.
    int lane, l32, hf, gi;
    int kaddr[4];        // K operand byte offset for k-step ks (rows l32, chunk 2·ks + hf)
    int vaddr[2][2];     // Vᵀ transpose-read byte offset for [dv tile dt][first/second 4 keys], k-step 0
    int ld_koff[LOADS];  // global byte offset (within a tile) of this lane's K loads
    int ld_voff[LOADS];  // same for V (K and V may have different row strides)
    int ld_lds[LOADS];   // LDS byte offset (within a tile) of those loads (wave-uniform)
    // Per-wave state.
    bf16x8 qop[QT][4];
    f32x16 oacc[QT][2];
    float mref[QT], lsum[QT];
    // Per-workgroup scalars.
    const char* kg;
    const char* vg;
    int kr, vr;  // row strides of K and V (elements)
    int L, wq0;
    KeyWindow win;
    // Per-wave key ranges: [wlo, whi) is needed by some query of the wave,
    // [flo, fhi) is legal for every query of the wave.
    int wlo, whi, flo, fhi;
    float c_log2;
    // Dropout: this lane's keep-bit rows (one per sub-block), and the words
    // of two consecutive tiles (keys k0 .. k0 + 127 of the even step's tile).
    const uint32_t* krow[QT];
    int kwords;
    u32x4 kwv[QT];

    // The keep words of tiles t and t + 1, one 16-byte load per row where all
    // four lie in the row (zero past its last word).  One load per lane for
    // two tiles keeps the cache traffic of the mask (each lane reads its own
    // row, 32 rows per instruction) at a quarter of single-word loads.
    __device__ void load_keep2(int t) {
        const int w0 = 2 * t;
        if (w0 + 4 <= kwords) {  // uniform
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) __builtin_memcpy(&kwv[qt], krow[qt] + w0, 16);
        } else {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int i = 0; i < 4; ++i) kwv[qt][i] = w0 + i < kwords ? krow[qt][w0 + i] : 0u;
        }
    }

    __device__ void issue_tile_load(int t, int buf) {
        const int k0 = t * BN;
        // buffer ranges end with the last legal row (L - k0 > 0 rows from k0 on)
        const int krr = STRIDED ? kr : D, vrr = STRIDED ? vr : D;
        const i32x4 rk = make_rsrc(kg + (size_t)k0 * krr * 2, rows_span(L - k0, krr, D, 2));
        const i32x4 rv = make_rsrc(vg + (size_t)k0 * vrr * 2, rows_span(L - k0, vrr, D, 2));
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            load16_to_lds(rk, lds + buf * 2 * TILE_BYTES + ld_lds[i], ld_koff[i]);
            load16_to_lds(rv, lds + buf * 2 * TILE_BYTES + TILE_BYTES + ld_lds[i], ld_voff[i]);
        }
    }

    // −∞ on the illegal logits of sub-block qt (tiles on a window edge or the
    // padding edge).  Register i of sub-tile kt is key
    // k0 + 32·kt + 8·(i/4) + 4·hf + i%4 of query wq0 + 32·qt + l32.
    __device__ void mask_block(int qt, int k0, f32x16 (&s)[2]) {
        const int qrow = wq0 + 32 * qt + l32;
        const int llo = win.lo(qrow) - k0 - 4 * hf;
        const int lhi = win.hi(qrow) - k0 - 4 * hf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 32 * kt + 8 * (i >> 2) + (i & 3);
                s[kt][i] = (off >= llo && off < lhi) ? s[kt][i] : -INFINITY;
            }
    }

    // P = 2^(s·c − m·c) = e^(scale·(s − m)) for sub-block qt (masked entries
    // give exactly 0), packed into the four bf16 B operands of Oᵀ += Vᵀ·Pᵀ.
    // Returns this lane's partial sum of the (bf16) weights.  k-step j takes
    // sub-tile j/2, registers 8·(j%2)..+7, i.e. for half-wave hf the keys
    // 16·j + 4·hf + [0..3] and 16·j + 8 + 4·hf + [0..3].
    __device__ float softmax_weights(float mc, const f32x16 (&s)[2], bf16x8 (&pb)[4]) {
        const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
        float l = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kt = j >> 1, vb = 8 * (j & 1);
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = exp2_hw(__builtin_fmaf(s[kt][vb + e], c_log2, -mc));
            const bf16x8 v = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
            pb[j] = v;
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), ones, l, false);
        }
        return l;
    }

    // One tile of math for both sub-blocks.  Every K operand read from LDS feeds
    // the Sᵀ products of both sub-blocks, and every Vᵀ operand both P·V products.
    // (The masking branch also bounds how far the compiler hoists the softmax
    // into the products, which keeps the wave at two per SIMD.)
    template <int BUF>
    __device__ void compute_tile(int k0) {
        const char* sk = lds + BUF * 2 * TILE_BYTES;
        const char* sv = sk + TILE_BYTES;

        // Sᵀ = K · Qᵀ over d = 64 (four k-steps of 16).
        f32x16 s[QT][2];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[qt][kt][i] = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(sk + kaddr[ks] + kt * 32 * 128);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) s[qt][kt] = mfma32x32x16_bf16(a, qop[qt][ks], s[qt][kt]);
            }

        // −∞ on illegal logits: tiles not wholly legal for every query of the wave.
        if (k0 < flo || k0 + BN > fhi) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) mask_block(qt, k0, s[qt]);
        }

        // Weights against the current reference maximum, without computing this
        // tile's maximum: if every lane's partial sum stays within SUM_LIMIT,
        // no weight exceeds it and the tile is done (the reference cancels in
        // Σ p·v / Σ p).  Otherwise — and on a wave's first tile, where there is
        // no reference yet — take the tile maxima, move the reference to them,
        // rescale Oᵀ and l, and recompute the weights (all ≤ 1).
        bf16x8 pb[QT][4];
        float lt[QT];
        bool unset = false;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) unset |= mref[qt] == -INFINITY;
        bool exact = __builtin_amdgcn_ballot_w64(unset) != 0;
        if (!exact) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) lt[qt] = softmax_weights(mref[qt] * c_log2, s[qt], pb[qt]);
            // overflow gives +inf, which fails the test; NaN (from NaN inputs) passes
            bool big = false;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) big |= lt[qt] > SUM_LIMIT;
            exact = __builtin_amdgcn_ballot_w64(big) != 0;
        }
        if (exact) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                float x = max3(s[qt][0][0], s[qt][0][1], s[qt][0][2]);
#pragma unroll
                for (int i = 3; i < 15; i += 2) x = max3(x, s[qt][0][i], s[qt][0][i + 1]);
                x = max3(x, s[qt][0][15], s[qt][1][0]);
#pragma unroll
                for (int i = 1; i < 15; i += 2) x = max3(x, s[qt][1][i], s[qt][1][i + 1]);
                x = max2(x, s[qt][1][15]);
                const float mnew = fmaxf(mref[qt], half_swap_max(x));
                // mref = −∞ (nothing accumulated yet) gives alpha = 0 on zeros;
                // mnew = −∞ (every key so far illegal) keeps alpha = 1.
                const float alpha = mnew == -INFINITY ? 1.f : exp2_hw((mref[qt] - mnew) * c_log2);
                mref[qt] = mnew;
                lsum[qt] *= alpha;
#pragma unroll
                for (int i = 0; i < 16; ++i) { oacc[qt][0][i] *= alpha; oacc[qt][1][i] *= alpha; }
                lt[qt] = softmax_weights((mnew == -INFINITY ? 0.f : mnew) * c_log2, s[qt], pb[qt]);
            }
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) lsum[qt] += lt[qt];
        // Dropout: zero the dropped weights of k-step j (keys 16·j + 4·hf +
        // [0..3] and + 8, bits of word j/2 from 16·(j%2) + 4·hf) after the row
        // sums have counted them.
        if constexpr (DROP) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t wd = kwv[qt][2 * BUF + (j >> 1)] >> (16 * (j & 1) + 4 * hf);
                    pb[qt][j] = keep_pairs(pb[qt][j], wd);
                }
        }

        // Oᵀ += Vᵀ · Pᵀ.  The Vᵀ operand lists the same keys as Pᵀ: two LDS
        // transpose reads, each giving 4 consecutive keys (rows 16·j + 4·hf +
        // [0..3], then + 8) of one dv column to every lane.
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(sv + vaddr[dt][0] + j * 16 * 128));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(sv + vaddr[dt][1] + j * 16 * 128));
                const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) oacc[qt][dt] = mfma32x32x16_bf16(va, pb[qt][j], oacc[qt][dt]);
            }
    }

    // One tile: start the next tile's HBM → LDS copy into the other buffer, do
    // this tile's math, then wait for the copy and meet at the barrier.  The
    // other buffer was last read before the previous barrier, so overwriting it
    // here is safe.
    template <int BUF>
    __device__ void step(int t, int tend) {
        if (t + 1 < tend) issue_tile_load(t + 1, BUF ^ 1);
        // Dropout: the even step (BUF 0) loads the keep words of its tile and
        // of the next one, which the odd step uses.
        if constexpr (DROP && BUF == 0) load_keep2(t);
        const int k0 = t * BN;
        if (k0 < whi && k0 + BN > wlo) {  // else: no query of this wave sees the tile
            compute_tile<BUF>(k0);
        }
        wait_vmem();
        __syncthreads();
    }
};

template <int NW, bool STRIDED, bool DROP>
__global__ __launch_bounds__(NW * 64) void sdpa_long_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    int BH, int H, int n, int m, float c_log2, int wl, int wr, int bottom_right,
    const int32_t* __restrict__ key_lens, int nqb, float* __restrict__ lse, Layout lay,
    const uint32_t* __restrict__ keep, float keep_scale) {
    using KT = LongKernel<NW, STRIDED, DROP>;
    __shared__ __attribute__((aligned(16))) char lds[2 * 2 * TILE_BYTES];
    KT k;
    k.lds = lds;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    k.lane = tid & 63;
    k.l32 = k.lane & 31;
    k.hf = k.lane >> 5;
    k.gi = k.lane & 15;
    k.c_log2 = c_log2;

    // Heaviest query blocks (latest under a causal mask) are dispatched first;
    // consecutive workgroups take different heads, so with B·h a multiple of 8
    // each XCD (workgroups are dealt round-robin over 8) always serves the same
    // heads and keeps their K/V in its own L2.
    const int g = blockIdx.x;
    const int bh = g % BH;
    const int qb = nqb - 1 - g / BH;
    const int b = bh / H;
    const int q0 = qb * KT::BM;

    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    k.L = L;
    k.win = KeyWindow{wl, wr, bottom_right ? L - n : 0, L};
    // Key tiles [tbeg, tend): the keys any query of the block may see.
    const int qlast = min(q0 + KT::BM, n) - 1;
    const int kbeg = k.win.lo(q0), kend = k.win.hi(qlast);
    const int tbeg = kbeg / BN;
    const int tend = kend > kbeg ? (kend + BN - 1) / BN : tbeg;

    const int hh = bh - b * H;
    const uint16_t* Qh = Q + (STRIDED ? head_offset(lay.q, b, hh) : (long long)bh * n * D);
    uint16_t* Oh = O + (STRIDED ? head_offset(lay.o, b, hh) : (long long)bh * n * D);
    k.kg = reinterpret_cast<const char*>(K + (STRIDED ? head_offset(lay.k, b, hh) : (long long)bh * m * D));
    k.vg = reinterpret_cast<const char*>(V + (STRIDED ? head_offset(lay.v, b, hh) : (long long)bh * m * D));
    k.kr = STRIDED ? lay.k.r : D;
    k.vr = STRIDED ? lay.v.r : D;
    const int qr = STRIDED ? lay.q.r : D, orr = STRIDED ? lay.o.r : D;
    k.wq0 = q0 + w * QW;
    {
        const int wlast = min(k.wq0 + QW, n) - 1;  // < wq0 for a wave past n: empty
        k.wlo = wlast < k.wq0 ? 0 : k.win.lo(k.wq0);
        k.whi = wlast < k.wq0 ? 0 : k.win.hi(wlast);
        k.flo = wlast < k.wq0 ? 0 : k.win.lo(wlast);
        k.fhi = wlast < k.wq0 ? 0 : k.win.hi(k.wq0);
    }

    // Per-lane LDS read offsets (tile-relative, buffer 0).
    {
        const int f = swz_f(k.l32);  // rows l32 and l32 + 32 share it
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) k.kaddr[ks] = k.l32 * 128 + (((2 * ks + k.hf) ^ f) << 4);
        // Rows 4·hf + gi/4 (+ 8 for the second read) of k-step 0; k-step j adds
        // 16·j rows, which leaves swz_f unchanged (it reads row bits 1..3).
        const int r0 = 4 * k.hf + (k.gi >> 2);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
            const int dv0 = 32 * dt + 16 * ((k.lane >> 4) & 1) + 4 * (k.gi & 3);
            k.vaddr[dt][0] = lds_swz(r0, dv0 >> 3) * 16 + (dv0 & 7) * 2;
            k.vaddr[dt][1] = lds_swz(r0 + 8, dv0 >> 3) * 16 + (dv0 & 7) * 2;
        }
    }
    // Per-lane load offsets: wave w's i-th 1 KiB load fills tile rows
    // 8·(w·LOADS + i) .. +7; lane ln lands in LDS slot (row ln/8, position ln%8),
    // which holds logical chunk (ln%8) ^ f(row).
#pragma unroll
    for (int i = 0; i < KT::LOADS; ++i) {
        const int row = 8 * (w * KT::LOADS + i) + (k.lane >> 3);
        const int pos = k.lane & 7;
        const int chunk = pos ^ swz_f(row);
        k.ld_koff[i] = row * k.kr * 2 + chunk * 16;
        k.ld_voff[i] = row * k.vr * 2 + chunk * 16;
        k.ld_lds[i] = 8 * (w * KT::LOADS + i) * 128;
    }

    // Qᵀ as the B operand: sub-block qt, lane holds query wq0 + 32·qt + l32,
    // d = 16·ks + 8·hf + [0..7].
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int qrow = k.wq0 + 32 * qt + k.l32;
        if (qrow < n) {
            const u32x4* src = reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * qr);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) k.qop[qt][ks] = __builtin_bit_cast(bf16x8, src[2 * ks + k.hf]);
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) k.qop[qt][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) { k.oacc[qt][0][i] = 0.f; k.oacc[qt][1][i] = 0.f; }
        k.mref[qt] = -INFINITY;
        k.lsum[qt] = 0.f;
        if constexpr (DROP) {
            // rows past n read row n − 1 (their outputs are not stored)
            const int qrow = min(k.wq0 + 32 * qt + k.l32, n - 1);
            k.kwords = (m + 31) >> 5;
            k.krow[qt] = keep + ((size_t)bh * n + qrow) * k.kwords;
        }
    }

    if (tend > tbeg) {
        k.issue_tile_load(tbeg, 0);
        wait_vmem();
    }
    __syncthreads();
    int t = tbeg;
    for (; t + 1 < tend; t += 2) {
        k.template step<0>(t, tend);
        k.template step<1>(t + 1, tend);
    }
    if (t < tend) k.template step<0>(t, tend);

    // ---- Oᵀ / l and store.  Register i of oacc[qt][dt] is dv = 32·dt + 8·(i/4)
    // + 4·hf + i%4 of query wq0 + 32·qt + l32.
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int qrow = k.wq0 + 32 * qt + k.l32;
        const float ltot = half_swap_sum(k.lsum[qt]);
        // no legal key ⇒ zero row; a NaN sum (NaN legal inputs) stays NaN
        const float inv = ltot != 0.f ? (DROP ? keep_scale : 1.f) / ltot : 0.f;
        // ln Σ e^(scale·s) = scale·mref + ln l, with the reference the weights
        // were formed against: −∞ for a row with no legal key
        if (lse && k.hf == 0 && qrow < n) {
            const float mc = k.mref[qt] == -INFINITY ? 0.f : k.mref[qt] * k.c_log2;
            lse[(size_t)bh * n + qrow] = (mc + log2f(ltot)) * 0.6931471805599453f;
        }
        if (qrow < n) {
            uint16_t* dst = Oh + (size_t)qrow * orr;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int dv = 32 * dt + 8 * i4 + 4 * k.hf;
                    bf16x4 o;
                    o[0] = (__bf16)(k.oacc[qt][dt][4 * i4 + 0] * inv);
                    o[1] = (__bf16)(k.oacc[qt][dt][4 * i4 + 1] * inv);
                    o[2] = (__bf16)(k.oacc[qt][dt][4 * i4 + 2] * inv);
                    o[3] = (__bf16)(k.oacc[qt][dt][4 * i4 + 3] * inv);
                    *reinterpret_cast<bf16x4*>(dst + dv) = o;
                }
        }
    }
}

template <int NW>
hipError_t launch_long(const Args& a, hipStream_t stream) {
    const int BH = a.B * a.H;
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    const int nqb = (a.n + NW * QW - 1) / (NW * QW);
    const auto kernel = a.keep ? (a.strided ? sdpa_long_bf16<NW, true, true> : sdpa_long_bf16<NW, false, true>)
                               : (a.strided ? sdpa_long_bf16<NW, true, false> : sdpa_long_bf16<NW, false, false>);
    hipLaunchKernelGGL(kernel, dim3(nqb * BH), dim3(NW * 64), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.out, BH, a.H, a.n, a.m, c_log2, a.wl, a.wr, a.bottom_right,
                       a.key_lens, nqb, a.lse, a.lay, a.keep, a.keep_scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_long(const Args& a, hipStream_t stream) {
    // A window bounded on both sides and narrower than 2048 keys: 2 waves
    // (128 queries) per workgroup.  The workgroup streams the union of its
    // queries' windows, 64·NW + wl + wr keys, while each wave needs only
    // 64 + wl + wr of them; with 4 waves the other waves idle at the barrier
    // on a quarter of the tiles of a 512-key window.
    if (a.wl >= 0 && a.wr >= 0 && (long long)a.wl + a.wr < 2048) return launch_long<2>(a, stream);
    // Otherwise 4 waves (256 queries) per workgroup once there are enough query
    // blocks to fill the chip; 2 waves (128 queries) below that.
    const long long blocks4 = (long long)a.B * a.H * ((a.n + 4 * QW - 1) / (4 * QW));
    return blocks4 >= 1024 ? launch_long<4>(a, stream) : launch_long<2>(a, stream);
}

hipError_t launch_bf16(const Args& a0, hipStream_t stream) {
    Args a = a0;
    if (!a.strided) a.lay = dense_layout(a.H, a.n, a.m, a.d, a.dv);  // packed layout
    // n, m <= 64: the Table 3 width pairs, and attention dropout at d_k = d_v ∈ {32, 64, 128}
    if (short_bf16_fits(a)) return launch_bf16_short(a, stream);
    // attention dropout, longer: d_k = d_v ∈ {32, 64, 128}
    if (a.keep) return a.d == D ? launch_bf16_long(a, stream) : launch_bf16_width(a, stream);
    if (a.d != D || a.dv != D) return launch_bf16_width(a, stream);
    if (decode_bf16_fits(a)) return launch_bf16_decode(a, stream);
    return launch_bf16_long(a, stream);
}

}  // namespace sdpa
