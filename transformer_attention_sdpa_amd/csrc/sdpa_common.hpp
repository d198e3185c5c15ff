// Shared device-side vocabulary of the gfx950 attention kernels: vector types,
// MFMA wrappers, cross-half-wave reduction, bf16 packing and the argument block
// that the C ABI hands to the per-dtype launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The one head width the kernels support (d_k == d_v == 64, the pages' base and
// big models).
constexpr int kHeadDim = 64;

// Element strides of one [B, h, len, d] tensor whose last dimension is
// contiguous: element (b, head, i, j) sits at b·b_ + head·h + i·r + j.  Row
// strides are at least d and fit 32-bit byte offsets within a head (the C ABI
// checks both), so rows past a length are out of a buffer range that ends at
// that length's last row.
struct Strides {
    long long b, h;
    int r;
};
struct Layout {
    Strides q, k, v, o;
};
// [B, h, len, d] packed row-major, the layout of the plain entry points.
inline Layout dense_layout(int H, int n, int m, int dk, int dv) {
    return Layout{{(long long)H * n * dk, (long long)n * dk, dk},
                  {(long long)H * m * dk, (long long)m * dk, dk},
                  {(long long)H * m * dv, (long long)m * dv, dv},
                  {(long long)H * n * dv, (long long)n * dv, dv}};
}
__device__ __forceinline__ long long head_offset(const Strides& s, int b, int head) {
    return (long long)b * s.b + (long long)head * s.h;
}
// Bytes a buffer range needs to cover rows [0, len) of width d (esz bytes per
// element) at row stride r: up to the end of the last row.
__device__ __forceinline__ uint32_t rows_span(int len, int r, int d, int esz) {
    return len > 0 ? (uint32_t)(((long long)(len - 1) * r + d) * esz) : 0u;
}

// Everything a launcher needs; validated by the C ABI before any HIP call.
// The mask is a key window around each query's aligned position c_i (i, or
// i + L − n when bottom-right aligned): key j is legal iff j < L,
// j ≥ c_i − wl (wl ≥ 0) and j ≤ c_i + wr (wr ≥ 0); −1 leaves a side open.
// The decoder's causal mask is (wl, wr) = (−1, 0), top-left.
struct Args {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    int B, H, n, m;
    float scale;          // > 0, finite
    int wl, wr;           // window sides, >= -1
    int bottom_right;     // 0: c_i = i; 1: c_i = i + L - n
    const int32_t* key_lens;  // device int32[B] or nullptr
    // Optional: per query row, ln Σ_j exp(scale · q·k_j) over the legal keys
    // (−∞ for a row with none), fp32 [B, H, n]; bf16 kernels only.
    float* lse = nullptr;
    // Head widths d_k (d) and d_v (dv): 64 and 64 in every kernel; the other
    // pairs that width_supported lists in the bf16 kernels.
    int d = kHeadDim;
    int dv = kHeadDim;
    // Optional workspace for split-key decoder steps (decode_split_bytes), or nullptr.
    void* work = nullptr;
    size_t work_bytes = 0;
    // Attention dropout: keep-bit words [B, H, n, ⌈m/32⌉] (bit j mod 32 of word
    // ⌊j/32⌋ keeps weight (i, j)) and the factor of the kept weights, or nullptr.
    const uint32_t* keep = nullptr;
    float keep_scale = 1.f;
    // Element strides of q, k, v and out (dense_layout for the plain entry points).
    Layout lay{};
    // True when `lay` came from the caller (sdpa_forward_strided): the
    // latency-bound kernels then use runtime strides, else compile-time ones.
    bool strided = false;
};

// Legal key range [lo, hi) of query row i under the window of one batch
// element (key length L, shift = c_i − i).  Both ends are non-decreasing in i,
// so a block of consecutive queries needs keys [lo(first), hi(last)) and every
// key in [lo(last), hi(first)) is legal for all of them.
// Both results lie in [0, L] (computed in 64 bits: i + shift + wr can pass 2^31).
struct KeyWindow {
    int wl, wr, shift, L;
    __device__ __forceinline__ int lo(int i) const {
        if (wl < 0) return 0;
        const long long c = (long long)i + shift - wl;
        return c <= 0 ? 0 : (c >= L ? L : (int)c);
    }
    __device__ __forceinline__ int hi(int i) const {
        if (wr < 0) return L;
        const long long c = (long long)i + shift + wr + 1;
        return c <= 0 ? 0 : (c >= L ? L : (int)c);
    }
    // The same in 32 bits, for kernels whose n and m are at most 64: the C ABI
    // caps each window side at n + m, so nothing here can pass 2^31.
    __device__ __forceinline__ int lo32(int i) const { return wl < 0 ? 0 : min(L, max(0, i + shift - wl)); }
    __device__ __forceinline__ int hi32(int i) const {
        return wr < 0 ? L : min(L, max(0, i + shift + wr + 1));
    }
};

// The multi-head sublayer (bf16): projections, attention, output projection.
struct MhaArgs {
    const void* x_q;   // [B, n, d_model]
    const void* x_kv;  // [B, m, d_model]
    const void* w_q;   // [h·64, d_model]
    const void* w_k;   // [h·64, d_model]
    const void* w_v;   // [h·64, d_model]
    const void* w_o;   // [d_model, h·64]
    void* out;         // [B, n, d_model]
    void* workspace;   // mha_workspace_bytes(B, n, m, h) bytes
    int B, n, m, d_model, h;
    float scale;
    int wl, wr, bottom_right;
    const int32_t* key_lens;
    int hd = kHeadDim;  // head width d_k = d_v: 32, 64 or 128
};
size_t mha_workspace_bytes(int B, int n, int m, int h, int hd);

// The gradient of Eq. (1) (bf16 or fp32): dQ, dK, dV from Q, K, V, the
// forward output O, its gradient dO and the forward pass's per-row log-sum-exp.
struct BwdArgs {
    const void* q;     // [B, H, n, 64]
    const void* k;     // [B, H, m, 64]
    const void* v;     // [B, H, m, 64]
    const void* out;   // [B, H, n, 64], the forward output
    const void* dout;  // [B, H, n, 64]
    const float* lse;  // [B, H, n]
    void* dq;          // [B, H, n, 64]
    void* dk;          // [B, H, m, 64]
    void* dv;          // [B, H, m, 64]
    void* workspace;   // bwd_workspace_bytes(B, H, n) bytes
    int B, H, n, m;
    float scale;
    int wl, wr, bottom_right;
    const int32_t* key_lens;
    int d = kHeadDim;  // head width d_k = d_v: 32, 64 or 128
    // Attention dropout of the forward pass (as in Args), or nullptr.
    const uint32_t* keep = nullptr;
    float keep_scale = 1.f;
};
size_t bwd_workspace_bytes(int B, int H, int n);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t stream);   // d_k = d_v = 64
hipError_t launch_mha_bf16(const MhaArgs& a, hipStream_t stream);

hipError_t launch_bf16(const Args& a, hipStream_t stream);        // picks one of the four below
hipError_t launch_bf16_width(const Args& a, hipStream_t stream);  // widths other than 64/64
hipError_t launch_bf16_wide(const Args& a, hipStream_t stream);   // d_k = d_v = 512
// bf16 head widths (d_k, d_v): equal widths 16, 32, 64, 128 or 512, or d_v = 64 with d_k = 16 or 32.
bool width_supported(int d_k, int d_v);
hipError_t launch_bf16_long(const Args& a, hipStream_t stream);   // any n, m
hipError_t launch_bf16_short(const Args& a, hipStream_t stream);  // n, m <= 64; d = 32, 64, 128
bool short_bf16_fits(const Args& a);
hipError_t launch_bf16_decode(const Args& a, hipStream_t stream);  // n <= 16, m > 64
bool decode_bf16_fits(const Args& a);
// Workspace the decoder-step kernel uses to split each head's keys over
// several workgroups (0: it would not split these sizes).
size_t decode_split_bytes(int B, int H, int n, int m);
hipError_t launch_f32(const Args& a, hipStream_t stream);        // picks one of the two below
hipError_t launch_f32_long(const Args& a, hipStream_t stream);   // any n, m
hipError_t launch_f32_short(const Args& a, hipStream_t stream);  // n, m <= 64
bool short_f32_fits(const Args& a);

// max(a, b, c) in one v_max3_f32 and max(a, b) in one v_max_f32.  Written as
// instructions because fmaxf on MFMA results is lowered with an extra
// NaN-quieting v_max per operand.  The compiler inserts no wait states between
// an MFMA and an inline-asm reader of its result (up to 19 are needed): every
// use here sits far enough behind its MFMA, which a CPU test checks in the
// gfx950 assembly of each kernel.
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Both halves of a wave64 combined: after the call every lane holds
// op(x[lane], x[lane ^ 32]).  v_permlane32_swap exchanges the upper 32 lanes
// of one operand with the lower 32 lanes of the other; with the same value
// in both, the pair it returns is {x[lane], x[lane ^ 32]} in some order.
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the transcendental unit (v_exp_f32); 2^(−∞) is exactly +0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x2_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// LDS layout of a 64-column bf16 tile (128-byte rows, 16-byte chunks).  Chunk
// c of row r sits at chunk position c ^ swz_f(r), where swz_f(r) is the 3-bit
// reversal of (r/2 mod 8).  gfx950's LDS serves 256 bytes (64 banks) per pass,
// so two rows share a pass when they have the same parity; the XOR keeps
//   * 16 consecutive rows read at one chunk (a 16-byte MFMA operand per lane,
//     16 lanes per pass) on 16 different bank groups, and
//   * the 32-byte runs that ds_read_b64_tr_b16 takes from 4 or 8 consecutive
//     rows (32 lanes per pass) on disjoint bank groups.
__device__ __forceinline__ int swz_f(int row) {
    return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}
__device__ __forceinline__ int lds_swz(int row, int chunk) { return row * 8 + (chunk ^ swz_f(row)); }

// Raw buffer resource over [base, base + nbytes): loads at offsets >= nbytes
// return zeros without touching memory (gfx9 descriptor, dword 3 = 0x00020000).
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t nbytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = (int32_t)(uint32_t)a;
    r[1] = (int32_t)(uint32_t)((a >> 32) & 0xffffu);
    r[2] = (int32_t)nbytes;
    r[3] = 0x00020000;
    return r;
}

// buffer_load_dwordx4 … lds: lane i's 16 bytes from rsrc + voffset land at
// LDS address lds + 16·i (lds must be wave-uniform); out-of-range lanes write
// zeros.  Asynchronous: wait with s_waitcnt vmcnt before reading the LDS.
extern "C" __device__ void sdpa_llvm_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds,
                                                     int size, int voffset, int soffset, int offset,
                                                     int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
__device__ __forceinline__ void load16_to_lds(i32x4 rsrc, void* lds, int voffset) {
    sdpa_llvm_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}
// Same with the non-temporal (streaming) hint, for data that is read exactly
// once: it does not linger in the caches, and a short kernel then ends sooner
// (measured on the sentence-length kernels).
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void load16_to_lds_nt(i32x4 rsrc, void* lds, int voffset) {
    sdpa_llvm_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0,
                              kCachePolicyNT);
}
// 16-byte global store with the non-temporal hint (outputs are written once).
__device__ __forceinline__ void store16_nt(void* p, u32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}
// Attention dropout: keep_pairs zeroes the elements of eight packed bf16
// values whose keep bit is 0; the bits of elements 0..3 are bits 0..3 of
// `nib`, those of elements 4..7 bits 8..11 (other bits are ignored).  Each
// 32-bit pair of elements gets its mask from two 16-bit lanes: the low lane
// holds `nib`, the high lane `nib` >> 1, so both bits of a pair sit at one
// position q; a packed 16-bit shift left by 15 − q and an arithmetic shift
// right by 15 then fill each lane with its bit.
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 keep_pairs(bf16x8 v, uint32_t nib) {
    u32x4 w = __builtin_bit_cast(u32x4, v);
    const s16x2 t = __builtin_bit_cast(s16x2, (nib & 0xFFFFu) | ((nib << 15) & 0xFFFF0000u));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const short q = p < 2 ? 2 * p : 2 * p + 4;  // bit position of element 2·p
        const s16x2 x = (t << (short)(15 - q)) >> (short)15;
        w[p] &= __builtin_bit_cast(uint32_t, x);
    }
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier without the release fence of __syncthreads (which waits
// for every outstanding global load, LDS DMA included).  It waits only for the
// wave's own LDS operations (lgkmcnt); LDS data written by buffer loads needs
// its own s_waitcnt vmcnt before the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ds_read_b64_tr_b16 written as an instruction.  Through the builtin, the
// compiler cannot tell which LDS bytes an in-flight buffer_load … lds writes,
// so it waits for every outstanding global load before the read, including
// the prefetch of the next tile into the other buffer.  Written here, the read
// carries no such wait; the caller must make sure the bytes it reads have
// landed, and must pass the results through tr_wait (s_waitcnt lgkmcnt(0))
// before using them.  lds_addr points into __shared__ memory.
__device__ __forceinline__ u32x2 ds_read_tr16_b64(const void* lds_addr) {
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_addr;
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
    return r;
}
// Waits for the LDS reads above and ties their results to the wait, so no use
// of them can be scheduled before it.
__device__ __forceinline__ void tr_wait(u32x2 (&x)[8]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                   "+v"(x[6]), "+v"(x[7]));
}

// Round-to-nearest-even float → bf16 of eight values (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

}  // namespace sdpa
