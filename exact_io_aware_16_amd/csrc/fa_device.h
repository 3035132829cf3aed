// Device helpers for the gfx950 attention kernels: vector types, the bf16
// matrix-core instruction, bf16 packing and cross-lane exchanges.
//
// Matrix-core layout used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l supplies row (l % 32), eight k values for half l / 32;
//   B (16 x 32): lane l supplies column (l % 32), the same eight k values;
//   C (32 x 32): lane l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + i%4
//                for its sixteen accumulators i = 0..15.
// Only the C layout is fixed by the hardware for our purposes: the k index of
// an (half, element) slot may be any bijection as long as A and B agree, and
// every kernel here picks that bijection to make its loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native vector for 16-byte loads/stores (HIP's uint4 struct is copied through
// memory by the compiler, which keeps staging arrays out of registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

// Value of lane (l ^ 32) for every lane l.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Wave-uniform "all lanes true".
__device__ __forceinline__ bool wave_all(bool p) { return __all(p); }

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}


// Column E (0..7) of two 8 x bf16 row chunks, packed as (row a, row b) in one
// dword: low half from a, high half from b (one v_perm_b32).
template <int E>
__device__ __forceinline__ uint32_t pack_col(const u32x4& a, const u32x4& b) {
    return __builtin_amdgcn_perm(b[E >> 1], a[E >> 1], (E & 1) ? 0x07060302u : 0x05040100u);
}

}  // namespace fa
