// Sentence-length attention forward (n, m <= 64), bf16, gfx950.
//
// The pages' point that self-attention is cheap while the sequence length n is
// below the representation width d (《精读 Attention Is All You Need：原始
// Transformer 论文》, Table 1 and the discussion after it) makes this regime
// bound by memory traffic and latency, not by arithmetic: one head is 4 × 8 KiB
// of bf16 and ≈0.5 MFLOP.  The kernel is therefore built to get every HBM read
// of a head in flight at once and to keep the dependent chain short:
//
//   * one workgroup per (batch, head): the whole head (≤ 64 keys) is a single
//     tile, so the softmax is an exact two-pass one with no running rescale;
//   * four waves of 16 queries each on v_mfma_f32_16x16x32_bf16, so each wave's
//     serial MFMA/softmax chain is a quarter of a head;
//   * Q, K and V move HBM → LDS with buffer_load_dwordx4 … lds; Q is issued
//     before the key length is known, K right after it with its buffer range
//     ending at the key length, so padded rows are never read (they arrive as
//     zeros); V, ranged the same way, is requested once Q and K have landed,
//     so grid-wide the score operands go first, and it arrives while the
//     scores and the softmax run;
//   * every load and the output store carry the non-temporal hint: each byte
//     is touched once, and with nothing left dirty or resident in the caches
//     the kernel's end costs less (it took about 1 µs off each launch at
//     64 × 8 heads of 64 × 64);
//   * the output goes through LDS so that each store instruction writes whole
//     128-byte rows;
//   * key tiles of 16 that no query of the wave may see (past the key length,
//     or outside the queries' key windows: after the diagonal when causal)
//     are skipped in both products, and only tiles that straddle the padding
//     edge or a window edge are masked;
//   * Sᵀ = K·Qᵀ and Oᵀ = Vᵀ·Pᵀ (transposed, as in the long kernel) so the row
//     max/sum are lane-local plus two half/quarter-wave exchanges, and Vᵀ comes
//     from LDS transpose reads (ds_read_b64_tr_b16).
//
// The head widths are template parameters: d_k (DK) sets the Q and K tiles and
// the score product, d_v (DV) the V tile, P·V and the output.  64 and 64 for
// the base and big models; the variants of the same page's Table 3: equal
// widths 16, 32 and 128 (rows (A) and (C)), and d_k = 16 or 32 against
// d_v = 64 (row (B)).  Only the number of k-steps, of output tiles and of
// loads per wave, and the LDS swizzles, depend on them; at d_k = 16 the score
// product runs on v_mfma_f32_16x16x16_bf16 (one k-step of 16).
//
// Same arithmetic contract as the long kernel: fp32 scores and softmax, −∞ on
// illegal logits (《Attention Is All You Need：注意力就是你所需要的一切》
// §3.2.3) — the keys outside each query's window (KeyWindow) and past the key
// length — weights rounded to bf16 for P·V with fp32 accumulation, output
// rounded once to bf16.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int MAXLEN = 64;   // n and m bound of this kernel
constexpr int QW = 16;       // queries per wave
constexpr int NW = 4;        // waves per workgroup (4 × 16 = 64 queries)
constexpr int NT = NW * 64;

// Tile rows hold D bf16 values, D/8 chunks of 16 bytes; chunk c of row r
// sits at position c ^ g(r), where g is chosen per width so that
//   * 16 consecutive rows read at one chunk (a 16-byte MFMA operand per lane,
//     16 lanes per 256-byte LDS read cycle) fall on 16 distinct bank groups,
//   * the 8 rows × 32 bytes one ds_read_b64_tr_b16 cycle takes (rows
//     4G + 0..3 for two adjacent G, 32 bytes of dv each) fall on 8 distinct
//     32-byte bank groups:
//     D = 64 (128-byte rows): g = 3-bit reversal of (r/2 mod 8) (lds_swz);
//     D = 32 (64-byte rows, four to 256 bytes): g = 2-bit reversal of (r/4 mod 4);
//     D = 128 (256-byte rows): g = 2·(r mod 8) + (r/8 mod 2);
//     D = 16 (32-byte rows, eight to 256 bytes): g = r/8 mod 2 (the 16 rows
//     of a read then cover two 256-byte passes at distinct chunks, and the 8
//     rows of a transpose-read cycle, aligned to 8, stay contiguous).
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
    if constexpr (D == 64) {
        return lds_swz(row, chunk);
    } else if constexpr (D == 16) {
        return row * 2 + (chunk ^ ((row >> 3) & 1));
    } else if constexpr (D == 32) {
        const int s = (row >> 2) & 3;
        return row * 4 + (chunk ^ (((s & 1) << 1) | (s >> 1)));
    } else {
        return row * 16 + (chunk ^ (((row & 7) << 1) | ((row >> 3) & 1)));
    }
}

// op over lanes {l, l^16, l^32, l^48}: the four 16-lane groups hold the four
// key quarters of one query column.
__device__ __forceinline__ float quad_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return half_swap_max(x);
}
__device__ __forceinline__ float quad_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    return half_swap_sum(x);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// k = 16: lane (l16, G) gives A[l16][4G .. 4G+3] and B[4G .. 4G+3][l16].
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// WINDOWED = false: no key window or the causal one (wl = −1, wr ∈ {−1, 0},
// top-left), whose legal keys start at 0; the general window costs this
// latency-bound kernel a few percent, so it gets its own instantiation.
// STRIDED = false: the packed [B, h, len, D] layout with compile-time strides
// (the runtime-stride arithmetic would sit on this latency-bound kernel's
// critical path); true: the strides of `lay`.
// DROP: attention dropout with keep-bit words [B·h, n, ⌈m/32⌉] (packed layout
// only): the dropped weights leave P·V but not the row sum, and the output is
// scaled by keep_scale.
template <int DK, int DV, bool WINDOWED, bool STRIDED, bool DROP>
__global__ __launch_bounds__(NT) void sdpa_short_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    int H, int n, int m, float c_log2, int wl, int wr, int bottom_right,
    const int32_t* __restrict__ key_lens, float* __restrict__ lse, Layout lay,
    const uint32_t* __restrict__ keep, float keep_scale) {
    constexpr int RBK = 2 * DK, RBV = 2 * DV;  // bytes per tile row
    constexpr int TILE_K = MAXLEN * RBK;       // Q and K tiles of 64 rows
    constexpr int TILE_V = MAXLEN * RBV;       // V tile (and the output staging)
    constexpr int CPRK = DK / 8, CPRV = DV / 8;  // 16-byte chunks per row
    constexpr int KS = DK / 32;                // k-steps of 32 of the score product (0: one of 16)
    constexpr int DT = DV / 16;                // 16-wide output tiles
    // 1 KiB loads per tensor, and per wave: a wave moves consecutive rows
    // (its own 16 when a tensor takes at least one load per wave); a tensor
    // of fewer loads is moved by the first waves.
    constexpr int NLK = RBK / 16, NLV = RBV / 16;
    constexpr int LPK = NLK >= NW ? NLK / NW : 1, LPV = NLV >= NW ? NLV / NW : 1;
    // K tile at 0, Q tile at TILE_K, V tile after both and after the output
    // staging, which reuses the start of LDS once the scores are done.
    constexpr int V_OFF = 2 * TILE_K > TILE_V ? 2 * TILE_K : TILE_V;
    __shared__ __attribute__((aligned(16))) char lds[V_OFF + TILE_V];
    const u32x4* sK = reinterpret_cast<const u32x4*>(lds);
    const u32x4* sQ = reinterpret_cast<const u32x4*>(lds + TILE_K);
    const char* sVb = lds + V_OFF;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int G = lane >> 4;  // 16-lane group 0..3

    const int bh = blockIdx.x;
    const int b = bh / H;
    const int hh = bh - b * H;
    const uint16_t* Qh = Q + (STRIDED ? head_offset(lay.q, b, hh) : (long long)bh * n * DK);
    const uint16_t* Kh = K + (STRIDED ? head_offset(lay.k, b, hh) : (long long)bh * m * DK);
    const uint16_t* Vh = V + (STRIDED ? head_offset(lay.v, b, hh) : (long long)bh * m * DV);
    uint16_t* Oh = O + (STRIDED ? head_offset(lay.o, b, hh) : (long long)bh * n * DV);
    const int qr = STRIDED ? lay.q.r : DK, kr = STRIDED ? lay.k.r : DK;
    const int vr = STRIDED ? lay.v.r : DV, orr = STRIDED ? lay.o.r : DV;

    // HBM → LDS with buffer_load_dwordx4 … lds, 1024 / (row bytes) rows per
    // 1 KiB load u (rows from that count times u); lane ln lands in LDS slot
    // (row ln / chunks per row, position ln % chunks per row), which holds the
    // chunk whose swizzled position that is (the swizzle is an XOR, its own
    // inverse).  Global byte offsets: row · (row stride) + chunk · 16, per
    // tensor.  kload / vload: this wave moves rows of Q and K / of V.
    const bool kload = NLK >= NW || w < NLK, vload = NLV >= NW || w < NLV;
    int q_off[LPK], k_off[LPK], kq_lds[LPK], v_off[LPV], v_lds[LPV];
#pragma unroll
    for (int i = 0; i < LPK; ++i) {
        const int u = NLK >= NW ? LPK * w + i : w;
        const int row = (1024 / RBK) * u + lane / CPRK;
        const int c16 = (swz<DK>(row, lane % CPRK) - row * CPRK) * 16;
        q_off[i] = row * qr * 2 + c16;
        k_off[i] = row * kr * 2 + c16;
        kq_lds[i] = u * 1024;
    }
#pragma unroll
    for (int i = 0; i < LPV; ++i) {
        const int u = NLV >= NW ? LPV * w + i : w;
        const int row = (1024 / RBV) * u + lane / CPRV;
        v_off[i] = row * vr * 2 + (swz<DV>(row, lane % CPRV) - row * CPRV) * 16;
        v_lds[i] = u * 1024;
    }
    // Q goes first, without waiting for the key length.  Then the key length,
    // then K (and V, below), whose buffer ranges stop at it: their padded rows
    // arrive as zeros without being read (a zero K row only gives a score the
    // mask discards; a zero V row meets weight 0 in P·V, and 0 · garbage must
    // not happen).
    const i32x4 rq = make_rsrc(Qh, rows_span(n, qr, DK, 2));
    if (kload) {
#pragma unroll
        for (int i = 0; i < LPK; ++i) load16_to_lds_nt(rq, lds + TILE_K + kq_lds[i], q_off[i]);
    }
    // Dropout: the keep words of this lane's query (keys 0..31, 32..63); rows
    // past n read row n − 1 (their outputs are not stored).
    uint32_t kw[2] = {0u, 0u};
    if constexpr (DROP) {
        const int kwords = (m + 31) >> 5;
        const uint32_t* krow = keep + ((size_t)bh * n + min(w * QW + (lane & 15), n - 1)) * kwords;
        kw[0] = krow[0];
        kw[1] = kwords > 1 ? krow[1] : 0u;
    }
    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    const i32x4 rk = make_rsrc(Kh, rows_span(L, kr, DK, 2));
    if (kload) {
#pragma unroll
        for (int i = 0; i < LPK; ++i) load16_to_lds_nt(rk, lds + kq_lds[i], k_off[i]);
    }

    // Key tiles [kt0, nkt) hold every key some query of this wave may see;
    // keys in [flo, fhi) are legal for all of its queries.  Computed while Q
    // and K are in flight (the empty asm keeps them there).
    const int q = w * QW + l16;
    const int wfirst = w * QW, wlast = min(w * QW + QW, n) - 1;
    int kt0, nkt, flo, fhi, llo, lhi;
    if constexpr (WINDOWED) {
        const KeyWindow win{wl, wr, bottom_right ? L - n : 0, L};
        const int wlo = win.lo32(wfirst), whi = win.hi32(wlast);
        kt0 = wlo >> 4;
        nkt = whi > wlo ? (whi + 15) >> 4 : kt0;
        flo = win.lo32(wlast);
        fhi = win.hi32(wfirst);
        // Legal keys of this lane's query: [lo, hi).  Register r of tile kt is
        // key 16·kt + 4·G + r, so the test is llo <= 16·kt + r < lhi.
        llo = win.lo32(q) - 4 * G;
        lhi = win.hi32(q) - 4 * G;
        asm volatile("" : "+s"(kt0), "+s"(nkt), "+s"(flo), "+s"(fhi), "+v"(llo), "+v"(lhi));
    } else {
        const bool causal = wr == 0;  // keys [0, L), or [0, min(L, i + 1)) when causal
        kt0 = 0;
        nkt = causal ? min((L + 15) >> 4, w + 1) : (L + 15) >> 4;
        flo = 0;
        fhi = causal ? min(L, wfirst + 1) : L;
        llo = 0;
        lhi = (causal ? min(L, q + 1) : L) - 4 * G;
        asm volatile("" : "+s"(nkt), "+s"(fhi), "+v"(lhi));
    }
    // V is requested only once this wave's Q and K rows have landed: across
    // the grid, every workgroup's Q and K then reach HBM ahead of V traffic,
    // which the scores do not need.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // (the keep words are in too: any wait the compiler adds for them goes
    // here, ahead of the V requests, not behind them)
    if constexpr (DROP) asm volatile("" : "+v"(kw[0]), "+v"(kw[1]));
    const i32x4 rv = make_rsrc(Vh, rows_span(L, vr, DV, 2));
    if (vload) {
#pragma unroll
        for (int i = 0; i < LPV; ++i) load16_to_lds_nt(rv, lds + V_OFF + v_lds[i], v_off[i]);
    }
    lds_barrier();
    const bool active = w * QW < n;  // this wave has queries (n < 64 leaves some idle)

    // Qᵀ as the B operand: lane holds query q, d = 32·ks + 8·G + [0..7]
    // (d_k = 16: d = 4·G + [0..3], half G mod 2 of chunk G / 2).
    bf16x8 qop[KS > 0 ? KS : 1];
    s16x4 qop16;
    if constexpr (KS > 0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = __builtin_bit_cast(bf16x8, sQ[swz<DK>(q, 4 * ks + G)]);
    } else {
        qop16 = *reinterpret_cast<const s16x4*>(lds + TILE_K + swz<16>(q, G >> 1) * 16 + (G & 1) * 8);
    }


    // Sᵀ = K · Qᵀ: register r of tile kt is key 16·kt + 4·G + r.
    f32x4 s[4];
    bf16x8 pb[2];
    float l = 0.f;
    if (active) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            s[kt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (kt >= kt0 && kt < nkt) {  // uniform
                const int krow = 16 * kt + l16;
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (KS > 0) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 a = __builtin_bit_cast(bf16x8, sK[swz<DK>(krow, 4 * ks + G)]);
                        acc = mfma16(a, qop[ks], acc);
                    }
                } else {
                    const s16x4 a = *reinterpret_cast<const s16x4*>(lds + swz<16>(krow, G >> 1) * 16 + (G & 1) * 8);
                    acc = mfma16k16(a, qop16, acc);
                }
                if (16 * kt < flo || 16 * kt + 16 > fhi) {  // uniform: tile has illegal keys
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (WINDOWED) {
                            // llo <= off < lhi as one unsigned compare
                            const unsigned rel = (unsigned)(16 * kt + r - llo);
                            acc[r] = rel < (unsigned)(lhi - llo) ? acc[r] : -INFINITY;
                        } else {
                            acc[r] = (16 * kt + r < lhi) ? acc[r] : -INFINITY;
                        }
                    }
                }
                s[kt] = acc;
            }
        }
        float mx = max3(max3(s[0][0], s[0][1], s[0][2]), max3(s[0][3], s[1][0], s[1][1]),
                        max3(s[1][2], s[1][3], s[2][0]));
        mx = max3(mx, max3(s[2][1], s[2][2], s[2][3]), max3(s[3][0], s[3][1], s[3][2]));
        mx = quad_max(max2(mx, s[3][3]));
        const float mc = (mx == -INFINITY ? 0.f : mx) * c_log2;  // no (−∞) − (−∞)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = (kt >= kt0 && kt < nkt) ? exp2_hw(__builtin_fmaf(s[kt][r], c_log2, -mc))
                                                        : 0.f;
                s[kt][r] = p;
                l += p;
            }
        l = quad_sum(l);
        // ln Σ e^(scale·s) = (mc + log2 l)·ln 2: −∞ for a row with no legal key
        if (lse && G == 0 && q < n) lse[(size_t)bh * n + q] = (mc + log2f(l)) * 0.6931471805599453f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            pb[j] = to_bf16x8(s[2 * j][0], s[2 * j][1], s[2 * j][2], s[2 * j][3],
                              s[2 * j + 1][0], s[2 * j + 1][1], s[2 * j + 1][2], s[2 * j + 1][3]);
            // Dropout, after the row sum: slot e of pb[j] is key 32·j + 4·G + e
            // (e < 4) or 32·j + 16 + 4·G + (e − 4), bit 4·G + e or 16 + 4·G +
            // (e − 4) of word j.
            if constexpr (DROP) {
                const uint32_t wd = kw[j] >> (4 * G);
                pb[j] = keep_pairs(pb[j], (wd & 0xFu) | ((wd >> 8) & 0xF00u));
            }
        }
    }
    wait_vmem();  // V in
    lds_barrier();
    if (!active) return;

    // Oᵀ = Vᵀ · Pᵀ: k-step j covers keys 32·j + 4·G + [0..3] (slots 0..3, from
    // tile 2j) and 32·j + 16 + 4·G + [0..3] (slots 4..7, from tile 2j+1).
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const char* vb = sVb;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (2 * j >= nkt || 2 * j + 1 < kt0) continue;  // uniform: all these weights are zero
        const int r0 = 32 * j + 4 * G + (l16 >> 2);
        const int r1 = r0 + 16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int dv0 = 16 * dt + 4 * (l16 & 3);
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(vb + swz<DV>(r0, dv0 >> 3) * 16 + (dv0 & 7) * 2));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(vb + swz<DV>(r1, dv0 >> 3) * 16 + (dv0 & 7) * 2));
            o[dt] = mfma16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb[j], o[dt]);
        }
    }

    // Register r of o[dt] is dv = 16·dt + 4·G + r of query q.  The wave's 16
    // output rows go through its own 16 rows of a d_v-wide tile at the start
    // of LDS (the K and Q tiles, free since the barrier above) so that every
    // store instruction writes whole rows, 16 bytes a lane.
    {
        // no legal key ⇒ zero row; a NaN sum (NaN legal inputs) stays NaN
        const float inv = l != 0.f ? (DROP ? keep_scale * __builtin_amdgcn_rcpf(l) : __builtin_amdgcn_rcpf(l)) : 0.f;
        char* ob = lds + w * QW * RBV;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            bf16x4 ov;
            ov[0] = (__bf16)(o[dt][0] * inv);
            ov[1] = (__bf16)(o[dt][1] * inv);
            ov[2] = (__bf16)(o[dt][2] * inv);
            ov[3] = (__bf16)(o[dt][3] * inv);
            *reinterpret_cast<bf16x4*>(ob + swz<DV>(l16, 2 * dt + (G >> 1)) * 16 + (G & 1) * 8) = ov;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int SPW = QW * CPRV;  // 16-byte pieces of the wave's rows
#pragma unroll
        for (int i = 0; i < (SPW + 63) / 64; ++i) {
            const int id = lane + 64 * i;
            const int row = id / CPRV, c = id % CPRV;
            const int qq = w * QW + row;
            if (SPW % 64 == 0 || id < SPW) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(ob + swz<DV>(row, c) * 16);
                if (qq < n) store16_nt(Oh + (size_t)qq * orr + 8 * c, x);
            }
        }
    }
}

}  // namespace

bool short_bf16_fits(const Args& a) {
    if (a.n > MAXLEN || a.m > MAXLEN) return false;
    if (a.d == a.dv) return a.d == 16 || a.d == 32 || a.d == 64 || a.d == 128;
    return a.dv == 64 && (a.d == 16 || a.d == 32);
}

namespace {
template <int DK, int DV>
hipError_t launch_short(const Args& a, hipStream_t stream) {
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    const bool windowed = a.wl >= 0 || a.wr > 0 || a.bottom_right;
    auto kernel = a.strided ? (windowed ? sdpa_short_bf16<DK, DV, true, true, false> : sdpa_short_bf16<DK, DV, false, true, false>)
                            : (windowed ? sdpa_short_bf16<DK, DV, true, false, false> : sdpa_short_bf16<DK, DV, false, false, false>);
    if constexpr (DK == DV && DK >= 32) {  // the widths attention dropout takes; packed layout
        if (a.keep) {
            if (a.strided) return hipErrorInvalidValue;
            kernel = windowed ? sdpa_short_bf16<DK, DV, true, false, true> : sdpa_short_bf16<DK, DV, false, false, true>;
        }
    }
    if (a.keep && !(DK == DV && DK >= 32)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kernel, dim3(a.B * a.H), dim3(NT), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.out, a.H, a.n, a.m, c_log2, a.wl, a.wr, a.bottom_right,
                       a.key_lens, a.lse, a.lay, a.keep, a.keep_scale);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_bf16_short(const Args& a, hipStream_t stream) {
    if (a.d != a.dv) return a.d == 16 ? launch_short<16, 64>(a, stream) : launch_short<32, 64>(a, stream);
    if (a.d == 16) return launch_short<16, 16>(a, stream);
    if (a.d == 32) return launch_short<32, 32>(a, stream);
    if (a.d == 128) return launch_short<128, 128>(a, stream);
    return launch_short<64, 64>(a, stream);
}

}  // namespace sdpa
