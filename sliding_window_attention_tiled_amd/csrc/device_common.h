// device_common.h -- small device helpers shared by the HIP kernels of libswa.so.
#pragma once

#include <hip/hip_runtime.h>

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kEmptyMax = -1.0e30f;  // running max before any key was seen

// Workgroups are handed to the 8 XCDs round-robin by launch index.  This maps
// the launch index to a logical index such that each XCD receives one
// contiguous range of logical work items (neighbouring tiles share K/V rows,
// so they should share an L2).
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
    constexpr int X = 8;
    const int q = n / X, r = n % X;
    const int x = bid % X, i = bid / X;
    return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Value of lane l ^ 32, on the vector ALU (v_permlane32_swap exchanges the
// two 32-lane halves; no LDS round trip).  Whether the compiler swaps one
// register in place or two copies, lane l < 32 finds its partner in the
// second result and lane l >= 32 in the first.
__device__ __forceinline__ float lane_xor32(float x) {
    const unsigned b = __builtin_bit_cast(unsigned, x);
    const auto sw = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? sw[0] : sw[1]);
}

__device__ __forceinline__ float wave_max_xor32(float x) { return fmaxf(x, lane_xor32(x)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS transposing read: within each group of 16 lanes, lane j supplies the
// address of 4 consecutive 16-bit elements M[j][0..3]; lane i receives
// M[4e + i/4][i%4] for e = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
}

}  // namespace swa
