// Sentence-length attention forward (n, m <= 64), fp32, gfx950.
//
// Same computation as the other kernels — Eq. (1) of 《精读 Attention Is All You
// Need：原始 Transformer 论文》, softmax(Q Kᵀ·scale) V per (batch, head), with
// illegal logits at −∞ (《Attention Is All You Need：注意力就是你所需要的一切》
// §3.2.3) — in fp32 end to end: fp32 products on the matrix cores
// (v_mfma_f32_16x16x4_f32; gfx950 has no reduced-precision fp32 MFMA, so
// nothing is truncated), fp32 weights, fp32 output.
//
// Built like the bf16 sentence-length kernel: one workgroup per (batch, head),
// four waves of 16 queries, the whole head (≤ 64 keys) as one tile so the
// softmax is an exact two-pass one.  Q moves HBM → LDS (buffer_load … lds)
// before the key length is known, K right after it with its buffer range
// ending at the key length (padded rows are never read and arrive as zeros),
// and V, ranged the same way, once Q and K have landed; it arrives while the
// scores run.  Key tiles of 16 that no query of a wave may see (past the key
// length, or outside the queries' key windows, KeyWindow) are skipped.
//
// Products, transposed as elsewhere (each lane owns one query column):
//   Sᵀ (16 keys × 16 queries) = K · Qᵀ, 16 k-steps of 4; in k-step ks the
//     16-lane group G contributes d = 16·G + ks (a permutation of the
//     contraction index), so each lane reads 16 consecutive floats of its K
//     row and of its Q row;
//   Oᵀ (16 dv × 16 queries) += Vᵀ · Pᵀ, one k-step per (key tile kt, r): group
//     G contributes key 16·kt + 4·G + r, which is exactly the Sᵀ register
//     (kt, r) the lane already holds — Pᵀ never moves.  The 64 dv are spread
//     over four products so that one 16-byte LDS read feeds all four.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int D = kHeadDim;  // 64
constexpr int MAXLEN = 64;
constexpr int QW = 16;       // queries per wave
constexpr int NW = 4;
constexpr int NT = NW * 64;
constexpr int ROW = D * 4;   // 256-byte rows
constexpr int TILE = MAXLEN * ROW;  // 16 KiB

// fp32 tile in LDS: 16 chunks of 16 B per row; chunk c of row r sits at
// position c ^ (r mod 16), so 16 consecutive rows read at one chunk, and all
// 16 chunks of one row read by one 16-lane group, hit distinct banks.
__device__ __forceinline__ int f32_swz(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// op over lanes {l, l^16, l^32, l^48}.
__device__ __forceinline__ float quad_max_f(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return half_swap_max(max2(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_sum_f(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return half_swap_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// STRIDED as in the bf16 sentence-length kernel: compile-time strides for the
// packed layout, the runtime ones of `lay` otherwise.
template <bool STRIDED>
__global__ __launch_bounds__(NT) void sdpa_short_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, int H, int n, int m, float c_log2, int wl, int wr, int bottom_right,
    const int32_t* __restrict__ key_lens, float* __restrict__ lse, Layout lay) {
    // K tile at 0, Q at 16 KiB, V at 32 KiB.
    __shared__ __attribute__((aligned(16))) char lds[3 * TILE];
    const f32x4* sK = reinterpret_cast<const f32x4*>(lds);
    const f32x4* sQ = reinterpret_cast<const f32x4*>(lds + TILE);
    const f32x4* sV4 = reinterpret_cast<const f32x4*>(lds + 2 * TILE);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int G = lane >> 4;

    const int bh = blockIdx.x;
    const int b = bh / H;
    const int hh = bh - b * H;
    const float* Qh = Q + (STRIDED ? head_offset(lay.q, b, hh) : (long long)bh * n * D);
    const float* Kh = K + (STRIDED ? head_offset(lay.k, b, hh) : (long long)bh * m * D);
    const float* Vh = V + (STRIDED ? head_offset(lay.v, b, hh) : (long long)bh * m * D);
    float* Oh = O + (STRIDED ? head_offset(lay.o, b, hh) : (long long)bh * n * D);
    const int qr = STRIDED ? lay.q.r : D, kr = STRIDED ? lay.k.r : D;
    const int vr = STRIDED ? lay.v.r : D, orr = STRIDED ? lay.o.r : D;

    // Wave w moves tile rows 4·(4w + i) .. +3 (i = 0..3) of each tensor: one
    // 1 KiB load each; lane ln lands in LDS slot (row ln/16, position ln%16),
    // which holds logical chunk (ln%16) ^ (row mod 16).  Global byte offsets:
    // row · (row stride) + chunk · 16, per tensor.
    int q_off[4], k_off[4], v_off[4], ld_lds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (4 * w + i) + (lane >> 4);
        const int c16 = ((lane & 15) ^ (row & 15)) * 16;
        q_off[i] = row * qr * 4 + c16;
        k_off[i] = row * kr * 4 + c16;
        v_off[i] = row * vr * 4 + c16;
        ld_lds[i] = 4 * (4 * w + i) * ROW;
    }
    const i32x4 rq = make_rsrc(Qh, rows_span(n, qr, D, 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) load16_to_lds_nt(rq, lds + TILE + ld_lds[i], q_off[i]);
    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }
    const i32x4 rk = make_rsrc(Kh, rows_span(L, kr, D, 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) load16_to_lds_nt(rk, lds + ld_lds[i], k_off[i]);
    // V only once this wave's Q and K rows have landed (grid-wide, the score
    // operands reach HBM ahead of V); it arrives during the scores.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const i32x4 rv = make_rsrc(Vh, rows_span(L, vr, D, 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) load16_to_lds_nt(rv, lds + 2 * TILE + ld_lds[i], v_off[i]);
    lds_barrier();

    const int q = w * QW + l16;
    // Key tiles [kt0, nkt) hold every key some query of this wave may see.
    const KeyWindow win{wl, wr, bottom_right ? L - n : 0, L};
    const int wfirst = w * QW, wlast = min(w * QW + QW, n) - 1;
    const int wlo = win.lo32(wfirst), whi = win.hi32(wlast);
    const int kt0 = wlo >> 4;
    const int nkt = whi > wlo ? (whi + 15) >> 4 : kt0;
    const int qlo = win.lo32(q), qhi = win.hi32(q);  // this lane's legal keys
    const bool active = w * QW < n;

    // Qᵀ operand: d = 16·G + ks for k-step ks, i.e. Q[q][16G .. 16G+15].
    float qop[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 x = sQ[f32_swz(q, 4 * G + j)];
        qop[4 * j + 0] = x[0]; qop[4 * j + 1] = x[1]; qop[4 * j + 2] = x[2]; qop[4 * j + 3] = x[3];
    }

    // Sᵀ tiles; register r of tile kt is key 16·kt + 4·G + r of query q.
    f32x4 s[4];
    float l = 0.f, mc = 0.f;
    if (active) {
        // Key tiles in pairs (a tile of a pair past nkt is masked out below):
        // four independent accumulation chains keep the matrix pipe busy.
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
            s[2 * kp] = s[2 * kp + 1] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (2 * kp < nkt && 2 * kp + 1 >= kt0) {  // uniform
                f32x4 acc[2][2];
#pragma unroll
                for (int u = 0; u < 2; ++u) acc[u][0] = acc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const f32x4 a = sK[f32_swz(16 * (2 * kp + u) + l16, 4 * G + j)];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[u][j & 1] = mfma16x16x4(a[e], qop[4 * j + e], acc[u][j & 1]);
                    }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int kt = 2 * kp + u;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = 16 * kt + 4 * G + r;
                        const float x = acc[u][0][r] + acc[u][1][r];
                        s[kt][r] = (key >= qlo && key < qhi) ? x : -INFINITY;
                    }
                }
            }
        }
        float mx = max3(max3(s[0][0], s[0][1], s[0][2]), max3(s[0][3], s[1][0], s[1][1]),
                        max3(s[1][2], s[1][3], s[2][0]));
        mx = max3(mx, max3(s[2][1], s[2][2], s[2][3]), max3(s[3][0], s[3][1], s[3][2]));
        mx = quad_max_f(max2(mx, s[3][3]));
        mc = (mx == -INFINITY ? 0.f : mx) * c_log2;  // no (−∞) − (−∞)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2_hw(__builtin_fmaf(s[kt][r], c_log2, -mc));
                s[kt][r] = p;
                l += p;
            }
        l = quad_sum_f(l);
    }
    wait_vmem();  // V in
    lds_barrier();
    if (!active) return;

    // Oᵀ += Vᵀ · Pᵀ.  Output row i of product dt stands for dv = 4·f(i) + dt
    // with f(i) = 4·(i mod 4) + i/4, so A-operand lane l16 needs elements
    // 0..3 of chunk f(l16) of a V row: one 16-byte read serves all four
    // products.  Register r of o[dt] is then dv = 4·f(4·G + r) + dt
    // = 16·r + 4·G + dt of query q.
    f32x4 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int vchunk = 4 * (l16 & 3) + (l16 >> 2);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        if (kt < kt0 || kt >= nkt) continue;  // uniform; these weights are all zero
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f32x4 a = sV4[f32_swz(16 * kt + 4 * G + r, vchunk)];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[dt] = mfma16x16x4(a[dt], s[kt][r], o[dt]);
        }
    }

    if (q < n) {
        // 1/l to about an ulp: the hardware reciprocal refined by one Newton
        // step.  l = 0 (no legal key) gives a zero row; a NaN l (NaN among the
        // legal inputs) stays NaN.
        float inv = 0.f;
        if (l != 0.f) {
            inv = __builtin_amdgcn_rcpf(l);
            inv = __builtin_fmaf(__builtin_fmaf(-l, inv, 1.f), inv, inv);
        }
        // Store r writes dv 16·r + 4·G .. +3: the four 16-lane groups cover 64
        // contiguous bytes of each row per instruction.
        float* dst = Oh + (size_t)q * orr + 4 * G;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x4 ov;
            ov[0] = o[0][r] * inv;
            ov[1] = o[1][r] * inv;
            ov[2] = o[2][r] * inv;
            ov[3] = o[3][r] * inv;
            store16_nt(dst + 16 * r, __builtin_bit_cast(u32x4, ov));
        }
        // Natural-log log-sum-exp of the scaled logits: mc + log2 l in base 2,
        // −∞ for a query with no legal key (l = 0).
        if (lse && G == 0) lse[(size_t)bh * n + q] = (mc + log2f(l)) * 0.6931471805599453f;
    }
}

}  // namespace

bool short_f32_fits(const Args& a) { return a.n <= MAXLEN && a.m <= MAXLEN; }

hipError_t launch_f32_short(const Args& a, hipStream_t stream) {
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    hipLaunchKernelGGL(a.strided ? sdpa_short_f32<true> : sdpa_short_f32<false>, dim3(a.B * a.H), dim3(NT), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.out,
                       a.H, a.n, a.m, c_log2, a.wl, a.wr, a.bottom_right, a.key_lens, a.lse, a.lay);
    return hipGetLastError();
}

}  // namespace sdpa
