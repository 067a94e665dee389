// device_common.h -- small device helpers shared by the HIP kernels of libswa.so.
#pragma once

#include <hip/hip_runtime.h>

namespace swa {

// ---- debug build (-DSWA_DEBUG) ---------------------------------------------------
// SWA_DCHECK(cond) states an index contract of a kernel: a global row inside
// its tensor, a ring slot inside the ring, an LDS offset inside the tile, a
// device-side index (ring head, page id) inside its range before the kernel
// clamps it.  The debug build counts each failed check (one vector atomic add
// to a counter per translation unit) and carries on with the access, which the
// release code keeps in bounds anyway, so a broken contract is reported
// without faulting the device.  SWA_DEBUG_BARRIER() is an extra workgroup
// barrier at points where the release code relies on its own, weaker
// ordering: with it, phases that the release kernels overlap run one after
// the other, so a result that differs from the release build's in any bit
// points at a missing wait or barrier.  Both compile to nothing in release.
#ifdef SWA_DEBUG
static __device__ unsigned swa_debug_count;
#define SWA_DCHECK(cond)                                      \
    do {                                                      \
        if (!(cond)) atomicAdd(&::swa::swa_debug_count, 1u);  \
    } while (0)
#define SWA_DEBUG_BARRIER() __syncthreads()
// Defines a host function `name` that reads (and optionally clears) the
// counter of the translation unit it is placed in.
#define SWA_DEBUG_COUNTER_READER(name)                                                 \
    hipError_t name(unsigned* value, bool reset) {                                      \
        hipError_t e = hipMemcpyFromSymbol(value, HIP_SYMBOL(::swa::swa_debug_count),   \
                                           sizeof(unsigned), 0, hipMemcpyDeviceToHost); \
        if (e == hipSuccess && reset) {                                                 \
            const unsigned zero = 0;                                                    \
            e = hipMemcpyToSymbol(HIP_SYMBOL(::swa::swa_debug_count), &zero,            \
                                  sizeof(unsigned), 0, hipMemcpyHostToDevice);          \
        }                                                                               \
        return e;                                                                       \
    }
#else
#define SWA_DCHECK(cond) \
    do {                 \
    } while (0)
#define SWA_DEBUG_BARRIER() \
    do {                    \
    } while (0)
#endif

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
