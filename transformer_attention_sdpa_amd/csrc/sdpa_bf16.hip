// Fused single-pass attention forward for bf16 inputs on gfx950 (MI355X).
//
// Computes Eq. (1) of 《精读 Attention Is All You Need：原始 Transformer 论文》
// ("缩放点积注意力：点积为什么要缩放"), softmax(Q Kᵀ·scale) V, for every
// (batch, head) pair, with the decoder's illegal logits set to −∞ before the
// softmax (《Attention Is All You Need：注意力就是你所需要的一切》 §3.2.3) and key
// padding handled the same way.  Scores and softmax are fp32; the weights are
// rounded to bf16 (RNE) for the P·V product, which accumulates in fp32; the
// output is rounded once to bf16.
//
// Layout of the work.  One workgroup owns BM = NW·32 consecutive queries of one
// head; each of its NW waves owns 32 of them.  The keys of the head stream
// through LDS in tiles of 64 rows (K and V, 8 KiB each), and each wave keeps a
// running maximum and sum per query (online softmax), so no n×m score matrix
// ever exists.  Both products run on the matrix cores with
// v_mfma_f32_32x32x16_bf16, computed transposed:
//
//   Sᵀ (64 keys × 32 queries)  = K · Qᵀ          A = K rows from LDS, B = Qᵀ in VGPRs
//   Oᵀ (64 dv  × 32 queries) += Vᵀ · Pᵀ          A = Vᵀ via LDS transpose reads,
//                                                B = Pᵀ straight from the Sᵀ registers
//
// With the transposed form every lane holds one query's column, so the row
// max/sum of the softmax are lane-local plus one exchange between the two
// half-waves, and the per-query rescale of Oᵀ is a per-lane multiply.
//
// Causal blocks: a workgroup only visits key tiles up to its last query; a wave
// skips tiles that lie entirely after its queries; masking code only runs on
// tiles that straddle the diagonal or the padding edge.  Keys at or beyond the
// padding length are never read from HBM (their LDS rows are zero-filled).
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int D = kHeadDim;  // 64
constexpr int BN = 64;       // keys per LDS tile
constexpr int QW = 32;       // queries per wave

// 16-byte chunk c (0..7) of tile row r sits at chunk position c ^ (r & 7):
// rows that lanes read at the same column then fall in different banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <int NW>
__global__ __launch_bounds__(NW * 64) void sdpa_fwd_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    int BH, int H, int n, int m, float c_log2, int causal,
    const int32_t* __restrict__ key_lens, int nqb) {
    constexpr int NT = NW * 64;
    constexpr int CPT = (BN * D * 2 / 16) / NT;  // 16-byte chunks per thread per tile
    static_assert(CPT * NT * 16 == BN * D * 2, "tile must split evenly");

    __shared__ u32x4 sK[BN * 8];
    __shared__ u32x4 sV[BN * 8];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    // Heaviest query blocks (latest under a causal mask) are dispatched first.
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
    int kend = L;
    if (causal) kend = min(kend, q0 + NW * QW);
    const int ntiles = (kend + BN - 1) / BN;

    const size_t qbase = (size_t)bh * n * D;
    const size_t kvbase = (size_t)bh * m * D;

    // Qᵀ as the B operand: lane holds query l32, d = 16·ks + 8·hf + [0..7].
    const int qrow = q0 + w * QW + l32;
    bf16x8 qop[4];
    if (qrow < n) {
        const u32x4* src = reinterpret_cast<const u32x4*>(Q + qbase + (size_t)qrow * D);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qop[ks] = __builtin_bit_cast(bf16x8, src[2 * ks + hf]);
    } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qop[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }

    u32x4 rk[CPT], rv[CPT];
    auto gload = [&](int t) {
        const int k0 = t * BN;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            const int key = k0 + (c >> 3);
            if (key < L) {
                rk[i] = reinterpret_cast<const u32x4*>(K + kvbase + (size_t)key * D)[c & 7];
                rv[i] = reinterpret_cast<const u32x4*>(V + kvbase + (size_t)key * D)[c & 7];
            } else {
                rk[i] = u32x4{0, 0, 0, 0};
                rv[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto swrite = [&]() {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            const int idx = swz(c >> 3, c & 7);
            sK[idx] = rk[i];
            sV[idx] = rv[i];
        }
    };

    f32x16 oacc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) { oacc[0][i] = 0.f; oacc[1][i] = 0.f; }
    float mrun = -INFINITY;  // running max of raw scores q·k of this lane's query
    float lrun = 0.f;        // running sum of weights over this half-wave's keys

    const int wq_lo = q0 + w * QW;
    const int wq_hi = wq_lo + QW - 1;
    const int my_q = wq_lo + l32;

    if (ntiles > 0) gload(0);
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();  // every wave is done reading the previous tile
        swrite();
        __syncthreads();
        if (t + 1 < ntiles) gload(t + 1);  // next tile's HBM reads overlap this tile's math

        const int k0 = t * BN;
        if (causal && k0 > wq_hi) continue;  // tile lies entirely after this wave's queries

        // Sᵀ = K · Qᵀ over d = 64 (four k-steps of 16).
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
            const int krow = kt * 32 + l32;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, sK[swz(krow, 2 * ks + hf)]);
                s[kt] = mfma32x32x16_bf16(a, qop[ks], s[kt]);
            }
        }

        // −∞ on illegal logits: Sᵀ register i of lane (l32, hf) in sub-tile kt is
        // key k0 + 32·kt + 8·(i/4) + 4·hf + i%4 for query my_q.
        const bool need_mask = (k0 + BN > L) || (causal && k0 + BN - 1 > wq_lo);
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + kt * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (key >= L || (causal && key > my_q)) s[kt][i] = -INFINITY;
                }
        }

        float mt = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kt][i]);
        mt = half_swap_max(mt);
        const float mnew = fmaxf(mrun, mt);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;  // no (−∞) − (−∞)
        const float alpha = exp2_hw((mrun - muse) * c_log2);
        mrun = mnew;
        const float mc = muse * c_log2;
        lrun *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) { oacc[0][i] *= alpha; oacc[1][i] *= alpha; }

        // P = 2^(s·c − m·c) = e^(scale·(s − m)); masked entries give exactly 0.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = exp2_hw(__builtin_fmaf(s[kt][i], c_log2, -mc));
                s[kt][i] = p;
                lrun += p;
            }

        // Oᵀ += Vᵀ · Pᵀ in four k-steps of 16 keys.  k-step j takes Sᵀ sub-tile
        // j/2, registers 8·(j%2) .. +7; in tile rows that is, for half-wave hf,
        // keys kb + 4·hf + [0..3] and kb + 8 + 4·hf + [0..3] with kb = 16·j.
        // The Vᵀ operand must list the same keys: two LDS transpose reads, each
        // giving 4 consecutive keys of one dv column to every lane.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kt = j >> 1, vb = 8 * (j & 1);
            const bf16x8 pb = to_bf16x8(s[kt][vb + 0], s[kt][vb + 1], s[kt][vb + 2], s[kt][vb + 3],
                                        s[kt][vb + 4], s[kt][vb + 5], s[kt][vb + 6], s[kt][vb + 7]);
            const int kb = 16 * j;
            const int gi = lane & 15;
            const int r0 = kb + 4 * hf + (gi >> 2);
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                const int dv0 = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
                const int r1 = r0 + 8;
                const char* base = reinterpret_cast<const char*>(sV);
                const int off0 = swz(r0, dv0 >> 3) * 16 + (dv0 & 7) * 2;
                const int off1 = swz(r1, dv0 >> 3) * 16 + (dv0 & 7) * 2;
                typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(base + off0));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4*)(base + off1));
                const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[dt] = mfma32x32x16_bf16(va, pb, oacc[dt]);
            }
        }
    }

    // Oᵀ / l.  Register i of oacc[dt] is dv = 32·dt + 8·(i/4) + 4·hf + i%4 of query my_q.
    const float ltot = half_swap_sum(lrun);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;  // no legal key ⇒ zero row
    if (qrow < n) {
        uint16_t* dst = O + qbase + (size_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int dv = 32 * dt + 8 * i4 + 4 * hf;
                bf16x4 o;
                o[0] = (__bf16)(oacc[dt][4 * i4 + 0] * inv);
                o[1] = (__bf16)(oacc[dt][4 * i4 + 1] * inv);
                o[2] = (__bf16)(oacc[dt][4 * i4 + 2] * inv);
                o[3] = (__bf16)(oacc[dt][4 * i4 + 3] * inv);
                *reinterpret_cast<bf16x4*>(dst + dv) = o;
            }
    }
}

}  // namespace

hipError_t launch_bf16(const Args& a, hipStream_t stream) {
    const int BH = a.B * a.H;
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    if (a.n <= 64) {
        constexpr int NW = 2;
        const int nqb = (a.n + NW * QW - 1) / (NW * QW);
        hipLaunchKernelGGL(sdpa_fwd_bf16<NW>, dim3(nqb * BH), dim3(NW * 64), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (uint16_t*)a.out, BH, a.H, a.n, a.m, c_log2, a.causal, a.key_lens, nqb);
    } else {
        constexpr int NW = 4;
        const int nqb = (a.n + NW * QW - 1) / (NW * QW);
        hipLaunchKernelGGL(sdpa_fwd_bf16<NW>, dim3(nqb * BH), dim3(NW * 64), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (uint16_t*)a.out, BH, a.H, a.n, a.m, c_log2, a.causal, a.key_lens, nqb);
    }
    return hipGetLastError();
}

}  // namespace sdpa
