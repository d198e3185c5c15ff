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

// Head width this build supports (d_k == d_v == 64, the pages' base and big models).
constexpr int kHeadDim = 64;

// Everything a launcher needs; validated by the C ABI before any HIP call.
struct Args {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    int B, H, n, m;
    float scale;          // > 0, finite
    int causal;           // 0 or 1 (n == m when 1)
    const int32_t* key_lens;  // device int32[B] or nullptr
};

hipError_t launch_bf16(const Args& a, hipStream_t stream);
hipError_t launch_f32(const Args& a, hipStream_t stream);

// Both halves of a wave64 combined: after the call every lane holds
// op(x[lane], x[lane ^ 32]).  v_permlane32_swap exchanges the upper 32 lanes
// of one operand with the lower 32 lanes of the other; with the same value
// in both, the pair it returns is {x[lane], x[lane ^ 32]} in some order.
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// Round-to-nearest-even float → bf16 of eight values (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

}  // namespace sdpa
