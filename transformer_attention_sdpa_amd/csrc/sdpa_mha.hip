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
//      writes them straight into the [B, h, len, d] layout the attention
//      kernels read: the split into heads is the epilogue's store pattern;
//   2. the attention kernels of this library, on those tensors;
//   3. one projection launch for W^O whose token rows are gathered from the
//      [B, h, n, d] attention output: the Concat is its load pattern.
//
// The head width d is 32, 64 or 128 (the pages' model variants), with h·d a
// multiple of 64.
//
// Weights use the [out features, in features] layout, so that both MFMA
// operands are contiguous along the contraction: row i·64 + j of the Q weight
// is column j of W_i^Q, and W^O is stored as its transpose [d_model, h·64].
//
// The projection kernel computes Cᵀ = W · Xᵀ on v_mfma_f32_32x32x16_bf16: A =
// 32 weight rows (features), B = 32 token rows, so each lane ends up holding 4
// consecutive features of one token and stores them as one 8-byte write.  A
// workgroup of four waves (2 × 2) owns a tile of 64·MT tokens × 64·NT
// features; each wave 32·MT tokens × 32·NT features.  The contraction runs in
// stages of 64 inputs: per stage the workgroup's X and W rows (128 bytes
// each) are copied by buffer_load … lds straight into one of two LDS buffers,
// one stage ahead of the MFMAs, and every wave reads its operands from there.
// Loads use buffer ranges that end at the tensor, so token rows past M and
// feature rows past N read as zeros.
#include "sdpa_common.hpp"

namespace sdpa {
namespace {


enum { ROWS = 0, HEADS = 1 };

// One projection: C = X · Wᵀ over M tokens, N output features, K inputs.
// X is [M, K] row-major (ROWS) or the heads layout [M / len, K / hd, len, hd]
// (HEADS, token t = b·len + i, input k = head·hd + j); C is [M, N] (ROWS) or
// [M / len, N / hd, len, hd] (HEADS).  hd (the head width) is 32, 64 or 128.
struct ProjJob {
    const uint16_t* x;
    const uint16_t* w;  // [N, K]
    uint16_t* c;
    int M, N, K, len, hd;
};
struct ProjJobs {
    ProjJob job[3];
};

// ds_read_b128 written as an instruction: through a plain LDS load the
// compiler cannot tell which bytes an in-flight buffer_load … lds writes, and
// waits for all of them (the next stage's prefetch included) before the read.
// The caller waits with lgkm_wait before using the result.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E - 1.
template <int B, int E>
struct StaticFor {
    template <class F>
    __device__ __forceinline__ static void run(F&& f) {
        if constexpr (B < E) {
            f(std::integral_constant<int, B>{});
            StaticFor<B + 1, E>::run(f);
        }
    }
};
template <int N, int CNT>
__device__ __forceinline__ void lgkm_wait(u32x4 (&x)[N]) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(CNT));
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}

template <int AMODE, int CMODE, int MT, int NT>
__global__ __launch_bounds__(256) void proj_gemm_bf16(ProjJobs jobs) {
    constexpr int TM = 64 * MT, TN = 64 * NT;     // tokens × features per workgroup
    constexpr int XB = TM * 128, STAGE = (TM + TN) * 128;
    constexpr int NXI = TM / 32, NWI = TN / 32;  // LDS-DMA loads per wave per stage
    __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE];

    const ProjJob& J = jobs.job[blockIdx.z];
    const int t0 = blockIdx.x * TM;
    const int f0 = blockIdx.y * TN;
    if (t0 >= J.M || f0 >= J.N) return;  // uniform: this job has fewer tiles

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int K = J.K;
    const int nst = K / 64;

    // LDS-DMA: load u of wave w fills 8 rows (1 KB) of a stage's X or W tile,
    // rows 8·(w + 4u) .. +7; lane L writes row +L/8 at chunk position L%8,
    // which holds input chunk (L%8) ^ swz_f(row) of that row.
    const i32x4 rx = make_rsrc(J.x, (uint32_t)J.M * (uint32_t)K * 2u);
    const i32x4 rw = make_rsrc(J.w, (uint32_t)J.N * (uint32_t)K * 2u);
    uint32_t xo[NXI], wo[NWI];
    int xc[NXI];
#pragma unroll
    for (int u = 0; u < NXI; ++u) {
        const int r = 8 * (w + 4 * u) + (lane >> 3);
        const uint32_t c16 = (uint32_t)(((lane & 7) ^ swz_f(r)) * 16);
        const int t = t0 + r;
        if (AMODE == ROWS) {
            xo[u] = (uint32_t)t * (uint32_t)K * 2u + c16;
        } else {
            // row base of token t in the heads layout; the chunk's head and
            // offset inside it are added per stage (a stage may span heads)
            const int b = t / J.len, i = t - b * J.len;
            xo[u] = t < J.M ? ((uint32_t)(b * (K / J.hd)) * (uint32_t)J.len + (uint32_t)i) * (uint32_t)(J.hd * 2)
                            : 0xffffffffu;
            xc[u] = (int)c16 / 2;  // input offset of the chunk within a stage
        }
    }
#pragma unroll
    for (int u = 0; u < NWI; ++u) {
        const int r = 8 * (w + 4 * u) + (lane >> 3);
        wo[u] = (uint32_t)(f0 + r) * (uint32_t)K * 2u + (uint32_t)(((lane & 7) ^ swz_f(r)) * 16);
    }
    // Stage s: inputs 64·s .. +63.  ROWS: 128 bytes further along each row;
    // HEADS: input k = 64·s + the chunk's offset sits in head k / hd at k % hd.
    const uint32_t head_bytes = (uint32_t)J.len * (uint32_t)(J.hd * 2);
    const int hd_shift = J.hd == 32 ? 5 : (J.hd == 64 ? 6 : 7);
    auto xoff = [&](int u, int s) -> uint32_t {
        if (AMODE == ROWS) return xo[u] + (uint32_t)s * 128u;
        if (xo[u] == 0xffffffffu) return (uint32_t)J.M * (uint32_t)K * 2u;  // past the tensor: zeros
        const int k = 64 * s + xc[u];
        return xo[u] + (uint32_t)(k >> hd_shift) * head_bytes + (uint32_t)((k & (J.hd - 1)) * 2);
    };
    auto issue = [&](int s) {
        char* base = lds + (s & 1) * STAGE;
#pragma unroll
        for (int u = 0; u < NXI; ++u)
            load16_to_lds(rx, base + (w + 4 * u) * 1024, (int)xoff(u, s));
#pragma unroll
        for (int u = 0; u < NWI; ++u)
            load16_to_lds(rw, base + XB + (w + 4 * u) * 1024, (int)(wo[u] + (uint32_t)s * 128u));
    };

    // Operand reads: lane (l32, hf) reads row l32 of a 32-row block at input
    // chunk 2·ks + hf of k-step ks, i.e. at chunk position (2·ks + hf) ^ sw.
    const int wm = w & 1, wn = w >> 1;
    const int sw = swz_f(l32);
    const uint32_t lbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
    uint32_t ra[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ra[ks] = lbase + l32 * 128 + (((2 * ks + hf) ^ sw) * 16);
    constexpr int XOFF = 0;  // X rows of wave wm: 32·MT·wm + 32·i
    constexpr int WOFF = XB;

    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Two k-steps' operands per read batch: MT + NT reads each.
    constexpr int NR = 2 * (MT + NT);
    const uint32_t xo_w = wm * 32 * MT * 128, wo_w = wn * 32 * NT * 128;
    auto read_half = [&](uint32_t bufoff, auto hc, u32x4 (&v)[NR]) {
        constexpr int h = decltype(hc)::value;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t ax = ra[2 * h + q] + bufoff + xo_w, aw = ra[2 * h + q] + bufoff + wo_w;
            StaticFor<0, MT>::run([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                v[q * (MT + NT) + i] = ds_read16<XOFF + i * 4096>(ax);
            });
            StaticFor<0, NT>::run([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                v[q * (MT + NT) + MT + j] = ds_read16<WOFF + j * 4096>(aw);
            });
        }
    };
    auto mfma_half = [&](u32x4 (&v)[NR]) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = mfma32x32x16_bf16(__builtin_bit_cast(bf16x8, v[q * (MT + NT) + MT + j]),
                                                  __builtin_bit_cast(bf16x8, v[q * (MT + NT) + i]), acc[i][j]);
    };
    // The second half's reads are in flight while the first half's MFMAs run;
    // the scheduling barrier keeps the compiler from hoisting the second
    // wait above them.
    auto compute = [&](int s) {
        const uint32_t bufoff = (uint32_t)((s & 1) * STAGE);
        u32x4 v0[NR], v1[NR];
        read_half(bufoff, std::integral_constant<int, 0>{}, v0);
        read_half(bufoff, std::integral_constant<int, 1>{}, v1);
        lgkm_wait<NR, NR>(v0);
        mfma_half(v0);
        __builtin_amdgcn_sched_barrier(0);
        lgkm_wait<NR, 0>(v1);
        mfma_half(v1);
    };

    // Stage s sits in buffer s % 2.  Each wave waits for its own copies of
    // stage s (vmcnt), the barrier for everyone's; the barrier after the
    // reads frees the buffer for stage s + 2.
    constexpr int NI = NXI + NWI;
    issue(0);
    for (int s = 0; s + 1 < nst; ++s) {
        issue(s + 1);
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(NI) : "memory");
        compute(s);
        asm volatile("s_barrier" ::: "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    compute(nst - 1);

    // The output tile goes through LDS (the stage buffers are free once every
    // wave is past its last reads), so that the stores write 16 bytes a lane
    // along rows instead of 8-byte pieces of 32 different rows.  Register r of
    // acc[i][j] is feature 32·j + 8·(r/4) + 4·hf + r%4 (of the wave's feature
    // block) of token 32·i + l32 (of its token block); the tile row of a token
    // holds TN features in 8-byte pieces, piece s at s ^ (row mod 16).  LDS
    // takes 128 bytes of writes per cycle (16 lanes of 8 bytes) and they must
    // fall on distinct 8-byte positions modulo 128: the 16 rows one write
    // cycle covers then never collide.  16-byte chunk c of a row is read from
    // chunk c ^ ((row mod 16) / 2), its halves swapped when the row is odd.
    constexpr int CPR = TN / 8;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int row = 32 * MT * wm + 32 * i + l32;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int col = 32 * NT * wn + 32 * j + 8 * i4 + 4 * hf;
                bf16x4 o;
                o[0] = (__bf16)acc[i][j][4 * i4 + 0];
                o[1] = (__bf16)acc[i][j][4 * i4 + 1];
                o[2] = (__bf16)acc[i][j][4 * i4 + 2];
                o[3] = (__bf16)acc[i][j][4 * i4 + 3];
                *reinterpret_cast<bf16x4*>(lds + row * CPR * 16 + (((col >> 2) ^ (row & 15)) * 8)) = o;
            }
    }
    __syncthreads();
    // Thread t stores chunks t, t + 256, …: token row id / CPR, features 8·(id % CPR) .. +7.
#pragma unroll
    for (int k = 0; k < TM * CPR / 256; ++k) {
        const int id = tid + 256 * k;
        const int row = id / CPR, c = id % CPR;
        const int tok = t0 + row, f = f0 + 8 * c;
        const u32x4 y = *reinterpret_cast<const u32x4*>(lds + (row * CPR + (c ^ ((row & 15) >> 1))) * 16);
        const u32x4 x = (row & 1) ? u32x4{y[2], y[3], y[0], y[1]} : y;
        if (tok >= J.M || f >= J.N) continue;
        size_t dst;
        if (CMODE == ROWS) {
            dst = (size_t)tok * J.N + f;
        } else {
            // eight features inside one head: hd is 32, 64 or 128
            const int b = tok / J.len, ii = tok - b * J.len;
            dst = (((size_t)b * (J.N / J.hd) + f / J.hd) * J.len + ii) * J.hd + (f % J.hd);
        }
        *reinterpret_cast<u32x4*>(J.c + dst) = x;
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroup tile: the largest of 128 × 128, 128 × 64 and 64 × 64 (tokens ×
// features) that still gives at least two workgroups per compute unit, so
// that a second workgroup's loads overlap each one's MFMAs.
#ifndef SDPA_PROJ_TILE
#define SDPA_PROJ_TILE 0  // 0: by size; 1: 64 × 64; 2: 128 × 64; 3: 128 × 128
#endif
template <int AMODE, int CMODE>
hipError_t launch_proj(const ProjJobs& jobs, int njobs, int max_m, int n, hipStream_t stream) {
    auto tiles = [&](int tm, int tn) { return (long)((max_m + tm - 1) / tm) * ((n + tn - 1) / tn) * njobs; };
    int pick = SDPA_PROJ_TILE;
    if (pick == 0) pick = tiles(128, 128) >= 512 ? 3 : tiles(128, 64) >= 512 ? 2 : 1;
    if (pick == 3)
        hipLaunchKernelGGL((proj_gemm_bf16<AMODE, CMODE, 2, 2>), dim3((max_m + 127) / 128, (n + 127) / 128, njobs),
                           dim3(256), 0, stream, jobs);
    else if (pick == 2)
        hipLaunchKernelGGL((proj_gemm_bf16<AMODE, CMODE, 2, 1>), dim3((max_m + 127) / 128, (n + 63) / 64, njobs),
                           dim3(256), 0, stream, jobs);
    else
        hipLaunchKernelGGL((proj_gemm_bf16<AMODE, CMODE, 1, 1>), dim3((max_m + 63) / 64, (n + 63) / 64, njobs),
                           dim3(256), 0, stream, jobs);
    return hipGetLastError();
}

}  // namespace

size_t mha_workspace_bytes(int B, int n, int m, int h, int hd) {
    const size_t qo = (size_t)B * h * n * hd * 2, kv = (size_t)B * h * m * hd * 2;
    return 2 * align256(qo) + 2 * align256(kv);
}

hipError_t launch_mha_bf16(const MhaArgs& a, hipStream_t stream) {
    char* ws = static_cast<char*>(a.workspace);
    const int hd = a.hd;
    const size_t qo = align256((size_t)a.B * a.h * a.n * hd * 2);
    const size_t kv = align256((size_t)a.B * a.h * a.m * hd * 2);
    uint16_t* qh = reinterpret_cast<uint16_t*>(ws);
    uint16_t* kh = reinterpret_cast<uint16_t*>(ws + qo);
    uint16_t* vh = reinterpret_cast<uint16_t*>(ws + qo + kv);
    uint16_t* oh = reinterpret_cast<uint16_t*>(ws + qo + 2 * kv);
    const int hw = a.h * hd;

    // 1. Q, K, V projections into the heads layout.
    ProjJobs in{};
    in.job[0] = ProjJob{(const uint16_t*)a.x_q, (const uint16_t*)a.w_q, qh, a.B * a.n, hw, a.d_model, a.n, hd};
    in.job[1] = ProjJob{(const uint16_t*)a.x_kv, (const uint16_t*)a.w_k, kh, a.B * a.m, hw, a.d_model, a.m, hd};
    in.job[2] = ProjJob{(const uint16_t*)a.x_kv, (const uint16_t*)a.w_v, vh, a.B * a.m, hw, a.d_model, a.m, hd};
    hipError_t e = launch_proj<ROWS, HEADS>(in, 3, a.B * (a.n > a.m ? a.n : a.m), hw, stream);
    if (e != hipSuccess) return e;

    // 2. Attention over the B·h heads.
    Args att{qh, kh, vh, oh, a.B, a.h, a.n, a.m, a.scale, a.wl, a.wr, a.bottom_right, a.key_lens};
    att.d = hd;
    att.dv = hd;
    e = launch_bf16(att, stream);
    if (e != hipSuccess) return e;

    // 3. Concat(heads) · W^O, gathered from the heads layout.
    ProjJobs outj{};
    outj.job[0] = ProjJob{oh, (const uint16_t*)a.w_o, (uint16_t*)a.out, a.B * a.n, a.d_model, hw, a.n, hd};
    return launch_proj<HEADS, ROWS>(outj, 1, a.B * a.n, a.d_model, stream);
}

}  // namespace sdpa
