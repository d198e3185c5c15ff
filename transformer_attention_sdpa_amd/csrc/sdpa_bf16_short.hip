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
//   * Q goes straight from HBM into the B-operand registers; K and V are read
//     once per head, 16 bytes per lane, into LDS; rows at or past the key
//     length are not read (zero-filled);
//   * Sᵀ = K·Qᵀ and Oᵀ = Vᵀ·Pᵀ (transposed, as in the long kernel) so the row
//     max/sum are lane-local plus two half/quarter-wave exchanges, and Vᵀ comes
//     from LDS transpose reads (ds_read_b64_tr_b16).
//
// Same arithmetic contract as the long kernel: fp32 scores and softmax, −∞ on
// illegal logits (《Attention Is All You Need：注意力就是你所需要的一切》
// §3.2.3), weights rounded to bf16 for P·V with fp32 accumulation, output
// rounded once to bf16.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int D = kHeadDim;  // 64
constexpr int MAXLEN = 64;   // n and m bound of this kernel
constexpr int QW = 16;       // queries per wave
constexpr int NW = 4;        // waves per workgroup (4 × 16 = 64 queries)
constexpr int NT = NW * 64;

__device__ __forceinline__ int swz(int row, int chunk) { return lds_swz(row, chunk); }

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

__global__ __launch_bounds__(NT) void sdpa_short_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
    int H, int n, int m, float c_log2, int causal, const int32_t* __restrict__ key_lens) {
    __shared__ u32x4 sK[MAXLEN * 8];
    __shared__ u32x4 sV[MAXLEN * 8];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int G = lane >> 4;  // 16-lane group 0..3

    const int bh = blockIdx.x;
    const int b = bh / H;
    const size_t qbase = (size_t)bh * n * D;
    const size_t kvbase = (size_t)bh * m * D;

    // Qᵀ as the B operand: lane holds query q, d = 32·ks + 8·G + [0..7].
    const int q = w * QW + l16;
    bf16x8 qop[2];
    if (q < n) {
        const u32x4* src = reinterpret_cast<const u32x4*>(Q + qbase + (size_t)q * D);
        qop[0] = __builtin_bit_cast(bf16x8, src[G]);
        qop[1] = __builtin_bit_cast(bf16x8, src[4 + G]);
    } else {
        qop[0] = qop[1] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }

    int L = m;
    if (key_lens) {
        const int t = key_lens[b];
        L = t < 0 ? 0 : (t > m ? m : t);
    }

    // The head's legal K/V rows → LDS (rows ≥ L are zero: V rows enter P·V with
    // weight 0, and 0 · garbage must not happen).
#pragma unroll
    for (int i = 0; i < (MAXLEN * 8) / NT; ++i) {
        const int c = tid + i * NT;
        const int row = c >> 3;
        u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
        if (row < L) {
            kx = reinterpret_cast<const u32x4*>(K + kvbase + (size_t)row * D)[c & 7];
            vx = reinterpret_cast<const u32x4*>(V + kvbase + (size_t)row * D)[c & 7];
        }
        sK[swz(row, c & 7)] = kx;
        sV[swz(row, c & 7)] = vx;
    }
    __syncthreads();
    if (w * QW >= n) return;  // no queries for this wave (n < 64)

    // Sᵀ = K · Qᵀ: four 16-key tiles; register r of tile kt is key 16·kt + 4·G + r.
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int krow = 16 * kt + l16;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, sK[swz(krow, 4 * ks + G)]);
            s[kt] = mfma16(a, qop[ks], s[kt]);
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = 16 * kt + 4 * G + r;
            if (key >= L || (causal && key > q)) s[kt][r] = -INFINITY;
            mx = fmaxf(mx, s[kt][r]);
        }
    mx = quad_max(mx);
    const float mc = (mx == -INFINITY ? 0.f : mx) * c_log2;  // no (−∞) − (−∞)
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = exp2_hw(__builtin_fmaf(s[kt][r], c_log2, -mc));
            s[kt][r] = p;
            l += p;
        }
    l = quad_sum(l);

    // Oᵀ = Vᵀ · Pᵀ: k-step j covers keys 32·j + 4·G + [0..3] (slots 0..3, from
    // tile 2j) and 32·j + 16 + 4·G + [0..3] (slots 4..7, from tile 2j+1).
    f32x4 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const char* vb = reinterpret_cast<const char*>(sV);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const bf16x8 pb = to_bf16x8(s[2 * j][0], s[2 * j][1], s[2 * j][2], s[2 * j][3],
                                    s[2 * j + 1][0], s[2 * j + 1][1], s[2 * j + 1][2], s[2 * j + 1][3]);
        const int r0 = 32 * j + 4 * G + (l16 >> 2);
        const int r1 = r0 + 16;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int dv0 = 16 * dt + 4 * (l16 & 3);
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(vb + swz(r0, dv0 >> 3) * 16 + (dv0 & 7) * 2));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(vb + swz(r1, dv0 >> 3) * 16 + (dv0 & 7) * 2));
            o[dt] = mfma16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb, o[dt]);
        }
    }

    // Register r of o[dt] is dv = 16·dt + 4·G + r of query q.
    if (q < n) {
        const float inv = l > 0.f ? 1.f / l : 0.f;  // no legal key ⇒ zero row
        uint16_t* dst = O + qbase + (size_t)q * D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            bf16x4 ov;
            ov[0] = (__bf16)(o[dt][0] * inv);
            ov[1] = (__bf16)(o[dt][1] * inv);
            ov[2] = (__bf16)(o[dt][2] * inv);
            ov[3] = (__bf16)(o[dt][3] * inv);
            *reinterpret_cast<bf16x4*>(dst + 16 * dt + 4 * G) = ov;
        }
    }
}

}  // namespace

bool short_bf16_fits(const Args& a) { return a.n <= MAXLEN && a.m <= MAXLEN; }

hipError_t launch_bf16_short(const Args& a, hipStream_t stream) {
    const float c_log2 = (float)((double)a.scale * 1.4426950408889634);  // scale·log2(e)
    hipLaunchKernelGGL(sdpa_short_bf16, dim3(a.B * a.H), dim3(NT), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (uint16_t*)a.out, a.H, a.n, a.m, c_log2, a.causal, a.key_lens);
    return hipGetLastError();
}

}  // namespace sdpa
