// The multi-head attention sublayer on gfx950 (bf16):
//
//   MultiHead(Q, K, V) = Concat(head_1, …, head_h) W^O,
//   head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V)
//
// (《精读 Attention Is All You Need：原始 Transformer 论文》 multi-head section;
// 《Attention Is All You Need：注意力就是你所需要的一切》 §3.2.2), as three
// launches on the caller's stream:
//
//   1. one projection launch computes Q, K and V (three jobs, blockIdx.z) and
//      writes them straight into the [B, h, len, 64] layout the attention
//      kernels read: the split into heads is the epilogue's store pattern;
//   2. the attention kernels of this library, on those tensors;
//   3. one projection launch for W^O whose token rows are gathered from the
//      [B, h, n, 64] attention output: the Concat is its load pattern.
//
// Weights use the [out features, in features] layout, so that both MFMA
// operands are contiguous along the contraction: row i·64 + j of the Q weight
// is column j of W_i^Q, and W^O is stored as its transpose [d_model, h·64].
//
// The projection kernel computes Cᵀ = W · Xᵀ on v_mfma_f32_32x32x16_bf16: A =
// 32 weight rows (features), B = 32 token rows, so each lane ends up holding 4
// consecutive features of one token and stores them as one 8-byte write.  A
// workgroup of four waves owns 128 tokens × 64 features (one head); each wave
// 32 tokens.  Operands come straight from HBM/L2 with buffer loads whose range
// ends at the tensor, so token rows past M read as zeros.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {

constexpr int HD = kHeadDim;  // 64
constexpr int TM = 128;       // tokens per workgroup
constexpr int TN = 64;        // features per workgroup

enum { ROWS = 0, HEADS = 1 };

// One projection: C = X · Wᵀ over M tokens, N output features, K inputs.
// X is [M, K] row-major (ROWS) or the heads layout [M / len, K / 64, len, 64]
// (HEADS, token t = b·len + i, input k = head·64 + j); C is [M, N] (ROWS) or
// [M / len, N / 64, len, 64] (HEADS).
struct ProjJob {
    const uint16_t* x;
    const uint16_t* w;  // [N, K]
    uint16_t* c;
    int M, N, K, len;
};
struct ProjJobs {
    ProjJob job[3];
};

extern "C" __device__ i32x4 sdpa_mha_buffer_load_v4i32(i32x4 rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

template <int AMODE, int CMODE>
__global__ __launch_bounds__(256) void proj_gemm_bf16(ProjJobs jobs) {
    const ProjJob& J = jobs.job[blockIdx.z];
    const int t0 = blockIdx.x * TM;
    const int f0 = blockIdx.y * TN;
    if (t0 >= J.M || f0 >= J.N) return;  // uniform: this job has fewer tiles

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int tok = t0 + 32 * w + l32;
    const int K = J.K;

    // Byte offsets of this lane's 16-byte operand at contraction index 0:
    // token tok, inputs 8·hf .. +7; weight row f0 + 32·ft + l32, same inputs.
    const i32x4 rx = make_rsrc(J.x, (uint32_t)((size_t)J.M * K * 2));
    const i32x4 rw = make_rsrc(J.w, (uint32_t)((size_t)J.N * K * 2));
    int xoff;
    int xhead_stride = 0;  // HEADS: bytes from one head's block to the next
    if (AMODE == ROWS) {
        xoff = tok * K * 2 + hf * 16;
    } else {
        const int b = tok / J.len, i = tok - b * J.len;
        xoff = ((b * (K / HD)) * J.len + i) * HD * 2 + hf * 16;
        xhead_stride = J.len * HD * 2;
        if (tok >= J.M) xoff = J.M * K * 2;  // past the tensor: reads zeros
    }
    const int woff0 = (f0 + l32) * K * 2 + hf * 16;
    const int woff1 = woff0 + 32 * K * 2;

    f32x16 acc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc[0][i] = 0.f; acc[1][i] = 0.f; }

    // 64 inputs per iteration (four k-steps of 16); K is a multiple of 64, so
    // in HEADS mode one iteration is exactly one head's block.
    for (int k0 = 0; k0 < K; k0 += 64) {
        bf16x8 xo[4], wo[2][4];
        const int xk = AMODE == ROWS ? xoff + k0 * 2 : xoff + (k0 / HD) * xhead_stride;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            xo[s] = __builtin_bit_cast(bf16x8, sdpa_mha_buffer_load_v4i32(rx, xk + 32 * s, 0, 0));
            wo[0][s] = __builtin_bit_cast(bf16x8,
                                          sdpa_mha_buffer_load_v4i32(rw, woff0 + k0 * 2 + 32 * s, 0, 0));
            wo[1][s] = __builtin_bit_cast(bf16x8,
                                          sdpa_mha_buffer_load_v4i32(rw, woff1 + k0 * 2 + 32 * s, 0, 0));
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            acc[0] = mfma32x32x16_bf16(wo[0][s], xo[s], acc[0]);
            acc[1] = mfma32x32x16_bf16(wo[1][s], xo[s], acc[1]);
        }
    }

    // Register r of acc[ft] is feature f0 + 32·ft + 8·(r/4) + 4·hf + r%4 of
    // token tok: four consecutive features per 8-byte store.
    if (tok >= J.M) return;
    size_t cbase;
    int chead_stride = 0;
    if (CMODE == ROWS) {
        cbase = (size_t)tok * J.N;
    } else {
        const int b = tok / J.len, i = tok - b * J.len;
        cbase = ((size_t)b * (J.N / HD) * J.len + i) * HD;
        chead_stride = J.len * HD;
    }
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int f = f0 + 32 * ft + 8 * i4 + 4 * hf;
            const size_t dst = CMODE == ROWS ? cbase + f
                                             : cbase + (size_t)(f / HD) * chead_stride + (f % HD);
            bf16x4 o;
            o[0] = (__bf16)acc[ft][4 * i4 + 0];
            o[1] = (__bf16)acc[ft][4 * i4 + 1];
            o[2] = (__bf16)acc[ft][4 * i4 + 2];
            o[3] = (__bf16)acc[ft][4 * i4 + 3];
            *reinterpret_cast<bf16x4*>(J.c + dst) = o;
        }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t mha_workspace_bytes(int B, int n, int m, int h) {
    const size_t qo = (size_t)B * h * n * HD * 2, kv = (size_t)B * h * m * HD * 2;
    return 2 * align256(qo) + 2 * align256(kv);
}

hipError_t launch_mha_bf16(const MhaArgs& a, hipStream_t stream) {
    char* ws = static_cast<char*>(a.workspace);
    const size_t qo = align256((size_t)a.B * a.h * a.n * HD * 2);
    const size_t kv = align256((size_t)a.B * a.h * a.m * HD * 2);
    uint16_t* qh = reinterpret_cast<uint16_t*>(ws);
    uint16_t* kh = reinterpret_cast<uint16_t*>(ws + qo);
    uint16_t* vh = reinterpret_cast<uint16_t*>(ws + qo + kv);
    uint16_t* oh = reinterpret_cast<uint16_t*>(ws + qo + 2 * kv);
    const int hw = a.h * HD;

    // 1. Q, K, V projections into the heads layout.
    ProjJobs in{};
    in.job[0] = ProjJob{(const uint16_t*)a.x_q, (const uint16_t*)a.w_q, qh, a.B * a.n, hw, a.d_model, a.n};
    in.job[1] = ProjJob{(const uint16_t*)a.x_kv, (const uint16_t*)a.w_k, kh, a.B * a.m, hw, a.d_model, a.m};
    in.job[2] = ProjJob{(const uint16_t*)a.x_kv, (const uint16_t*)a.w_v, vh, a.B * a.m, hw, a.d_model, a.m};
    const int mt = (a.B * (a.n > a.m ? a.n : a.m) + TM - 1) / TM;
    hipLaunchKernelGGL((proj_gemm_bf16<ROWS, HEADS>), dim3(mt, hw / TN, 3), dim3(256), 0, stream, in);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 2. Attention over the B·h heads.
    const Args att{qh, kh, vh, oh, a.B, a.h, a.n, a.m, a.scale, a.wl, a.wr, a.bottom_right, a.key_lens};
    e = launch_bf16(att, stream);
    if (e != hipSuccess) return e;

    // 3. Concat(heads) · W^O, gathered from the heads layout.
    ProjJobs outj{};
    outj.job[0] = ProjJob{oh, (const uint16_t*)a.w_o, (uint16_t*)a.out, a.B * a.n, a.d_model, hw, a.n};
    hipLaunchKernelGGL((proj_gemm_bf16<HEADS, ROWS>), dim3((a.B * a.n + TM - 1) / TM, a.d_model / TN, 1),
                       dim3(256), 0, stream, outj);
    return hipGetLastError();
}

}  // namespace sdpa
