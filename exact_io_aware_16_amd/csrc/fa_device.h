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

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row sums of a P^T fragment on the matrix cores.  A B operand laid out for
// the 32x32x16 MFMA (lane (n, h) = (l & 31, l >> 5) holding keys 8h..8h+7 of
// query n) is, read as the B operand of a 16x16x32 MFMA, lane l holding rows
// k = 8 (l >> 4) .. +7 of column l & 15: k-groups 0 and 2 belong to query
// n = l & 15 and groups 1 and 3 to query n + 16.  With this A operand (row 0
// selects groups 0 and 2, row 1 groups 1 and 3, every other entry 0), D[0][j]
// is the sum over the fragment's 16 keys for query j and D[1][j] for query
// j + 16; both sit in lane j (elements 0 and 1) of the 16x16 result.
__device__ __forceinline__ bf16x8 rowsum_selector(int lane) {
    const bool one = lane == 0 || lane == 32 || lane == 17 || lane == 49;
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (__bf16)(one ? 1.f : 0.f);
    return a;
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

// max / sum of x over the lane pair (l, l ^ 32), on v_permlane32_swap: the
// swap hands each lane both halves' values without going through LDS.
__device__ __forceinline__ float pair_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Wave-uniform "all lanes true".
__device__ __forceinline__ bool wave_all(bool p) { return __all(p); }

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// ---------------------------------------------------------------------------
// Dense LDS tiles written by direct-to-LDS loads (no padding possible: each
// load instruction fills 64 consecutive 16-byte slots).  Bank conflicts are
// avoided instead by an XOR swizzle of the 16-byte chunk index within a row:
// chunk c of row r lives at slot c ^ swz(r).  swz is chosen so that
//  * 16 consecutive rows at one chunk (a 16-byte row read by 16 lanes) land in
//    16 distinct bank quads, and
//  * 4 consecutive rows x 4 consecutive chunks (one transpose read of a
//    16-lane group) land in 16 distinct bank quads.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);   // 16 chunks (256 B) per row
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);             // 8 chunks (128 B) per row
}

template <int D>
__device__ __forceinline__ int swz_off(int r, int c) {
    return r * D + ((c ^ swz<D>(r)) << 3);
}

// ---------------------------------------------------------------------------
// Matrix-core operand fragments read from those tiles (row = key or query,
// d contiguous).
// ---------------------------------------------------------------------------

// A (or B) fragment of X itself: lane l gets X[r0 + l%32][c0 + 8*(l/32) .. +7]
// (one 16-byte read).
template <int D>
__device__ __forceinline__ bf16x8 frag_rows_swz(const uint16_t* X, int r0, int c0, int lane) {
    return *reinterpret_cast<const bf16x8*>(X + swz_off<D>(r0 + (lane & 31), (c0 >> 3) + (lane >> 5)));
}

// A fragment of X^T (rows of the fragment = columns of X, k = rows of X) from
// the same tile, with two ds_read_b64_tr_b16: lane l gets
// X[k0 + 8*(e/4) + 4*(l/32) + e%4][c0 + l%32] for e = 0..7.
// ds_read_b64_tr_b16 hands lane i of each 16-lane group element i%4 of the
// 8-byte chunks addressed by lanes 4j + i/4 (j = 0..3), i.e. it transposes a
// 4-row x 16-column block; each lane therefore addresses row k0 + 4*(l/32) +
// (l%16)/4 at column c0 + 16*((l/16)%2) + 4*(l%4).
template <int D>
__device__ __forceinline__ bf16x8 frag_tr_swz(const uint16_t* X, int k0, int c0, int lane) {
    const int t = lane & 15;
    const int row = k0 + (lane >> 5) * 4 + (t >> 2);
    const int col = c0 + ((lane >> 4) & 1) * 16 + (t & 3) * 4;
    const uint16_t* p0 = X + swz_off<D>(row, col >> 3) + (col & 7);
    const uint16_t* p1 = X + swz_off<D>(row + 8, col >> 3) + (col & 7);
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// s_waitcnt on outstanding vector-memory operations only (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// (batch, query head) of launch position j in [0, B*Hq) of a kernel whose
// workgroups run over (position, head) pairs: the query heads of one K/V
// group sit B*Hkv positions apart, so with B*Hkv a multiple of 8 they land on
// one XCD (workgroup w runs on XCD w mod 8, the dispatcher's round robin)
// and read their shared K/V head through that XCD's L2.  With Hq == Hkv this
// is b = j / Hq, h = j % Hq.
__device__ __forceinline__ void group_major_head(int j, int B, int Hq, int Hkv, int& b, int& h) {
    const int BK = B * Hkv, g = Hq / Hkv;
    const int gi = j / BK, bk = j % BK;
    b = bk / Hkv;
    h = (bk % Hkv) * g + gi;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}


}  // namespace fa
