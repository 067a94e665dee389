// bwd_global.hip -- the backward's share of the global tokens: every (query,
// key) pair attended through a global token and not through the band.
//
// With global tokens (aiqz.cc "Sliding window attention: Mistral", section
// "global attention tokens") a global query row attends every key (causal:
// every key up to itself) and every query row attends each global key (causal:
// those not after it).  The band passes of the backward cover the pairs of the
// band for every row, global rows included: P is rebuilt from the final lse
// and delta from the final out.  The remaining pairs, outside the band, are
//   E_row = {(i, j): i global, j not in band(i)}          (global rows)
//   E_col = {(i, g): i not global, g global, g not in band(i)}  (global keys)
// each with j <= i when causal.  They are few (at most 256 rows or keys per
// head), so these kernels work on the vector ALUs in float32, in the layout of
// the float32 backward: rows (or keys) of a workgroup spread over lanes, with
// tiles of 32 partners (keys, or query rows) staged in LDS.  The passes over all
// N rows or keys take 64 per workgroup, four lanes each; the passes whose items
// are the global tokens take kGlobalBwdItems per workgroup, sixteen lanes each,
// so that a few tokens still fill the workgroup.  Same chain rule as
// the band passes: dS = P (dP - delta), dq = scale sum dS k, dk = scale sum dS q,
// dv = sum P dout.
//   rows_dq    dq of global rows over E_row, per key chunk, float32 atomics
//   rows_dkdv  dk, dv of every key over E_row, read-modify-write
//   cols_dq    dq of non-global rows over E_col, read-modify-write
//   cols_dkdv  dk, dv of global keys over E_col, per row chunk, float32 atomics
//   add_dq / add_dkdv fold the atomic accumulators into dq / dk, dv.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "swa_kernels.h"

namespace swa {
namespace {

constexpr float kLog2eG = 1.4426950408889634f;
constexpr int TK = 32;     // partners per LDS tile
constexpr int ITEMS = 64;  // rows or keys per workgroup of the all-N passes
constexpr int NT = 256;    // threads per workgroup

template <typename T>
__device__ __forceinline__ f32x4 ld4(const T* p);
template <>
__device__ __forceinline__ f32x4 ld4<float>(const float* p) {
    return *(const f32x4*)p;
}
template <>
__device__ __forceinline__ f32x4 ld4<__bf16>(const __bf16* p) {
    const bf16x4 x = *(const bf16x4*)p;
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
template <typename T>
__device__ __forceinline__ void st4(T* p, f32x4 x);
template <>
__device__ __forceinline__ void st4<float>(float* p, f32x4 x) {
    *(f32x4*)p = x;
}
template <>
__device__ __forceinline__ void st4<__bf16>(__bf16* p, f32x4 x) {
    *(bf16x4*)p = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}

// j in the band of i: same residue class and (j - i) / d in [-wl, wr]
__device__ __forceinline__ bool in_band(const GlobalBwdParams& g, int i, int j) {
    const int diff = j - i;
    if (diff % g.dil != 0) return false;
    const int t = diff / g.dil;
    return t >= -g.wl && t <= g.wr;
}

// the pair is in E_row or E_col (the caller knows which side is global)
__device__ __forceinline__ bool extra_pair(const GlobalBwdParams& g, int i, int j) {
    return !in_band(g, i, j) && (!g.causal || j <= i);
}

// position x among the sorted global positions (LDS copy)?
__device__ __forceinline__ bool is_global(const int* gp, int n, int x) {
    int lo = 0, hi = n - 1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const int v = gp[mid];
        if (v == x) return true;
        if (v < x) lo = mid + 1;
        else hi = mid - 1;
    }
    return false;
}

__device__ __forceinline__ void copy_gpos(const GlobalBwdParams& g, int* gp) {
    for (int i = threadIdx.x; i < g.n_global; i += NT) gp[i] = g.gpos[i];
}

// sum over the LANES consecutive lanes of an item
template <int LANES>
__device__ __forceinline__ float item_sum(float x) {
#pragma unroll
    for (int m = 1; m < LANES; m <<= 1) x += __shfl_xor(x, m);
    return x;
}
__device__ __forceinline__ float quad_sum(float x) { return item_sum<4>(x); }

// ---- rows_dq: dq of global rows over E_row ------------------------------------
// grid: (b, hq, tile of kGlobalBwdItems global rows, key chunk).  Few rows per
// workgroup, so each row takes NT / kGlobalBwdItems lanes.
template <int D, typename T>
__global__ __launch_bounds__(NT) void rows_dq_kernel(const GlobalBwdParams g) {
    constexpr int LANES = NT / kGlobalBwdItems;
    constexpr int DQ = D / LANES;
    constexpr int PITCH = D + 4;
    __shared__ __attribute__((aligned(16))) float ks[TK * PITCH];
    __shared__ __attribute__((aligned(16))) float vs[TK * PITCH];
    const int tid = threadIdx.x, part = tid % LANES;
    int L = blockIdx.x;
    const int chunk = L % g.n_key_chunks;
    L /= g.n_key_chunks;
    const int rt = L % g.row_tiles;
    L /= g.row_tiles;
    const int hq = L % g.Hq;
    const int b = L / g.Hq;
    const int kvh = hq / g.group;
    const int gi = rt * kGlobalBwdItems + tid / LANES;
    const bool row_ok = gi < g.n_global;
    const int i = row_ok ? g.gpos[gi] : 0;

    float q[DQ], dq[DQ], acc[DQ];
    const size_t qo = (((size_t)b * g.N + i) * g.Hq + hq) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
        const f32x4 a = ld4<T>((const T*)g.q + qo + d);
        const f32x4 o = ld4<T>((const T*)g.dout + qo + d);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            q[d + e] = a[e];
            dq[d + e] = o[e];
            acc[d + e] = 0.f;
        }
    }
    const size_t lrow = ((size_t)b * g.Hq + hq) * g.N + i;
    const float lse2 = g.lse[lrow] * kLog2eG;
    const float dlt = g.delta[lrow];
    const int j0 = chunk * g.key_chunk;
    const int j1 = min(g.N, j0 + g.key_chunk);
    const T* kb = (const T*)g.k + ((size_t)b * g.N * g.Hkv + kvh) * D;
    const T* vb = (const T*)g.v + ((size_t)b * g.N * g.Hkv + kvh) * D;
    const size_t rs = (size_t)g.Hkv * D;

    for (int t0 = j0; t0 < j1; t0 += TK) {
        __syncthreads();
        for (int ci = tid; ci < TK * D / 4; ci += NT) {
            const int kk = ci / (D / 4), c4 = ci % (D / 4);
            const int j = min(t0 + kk, j1 - 1);
            *(f32x4*)(ks + kk * PITCH + c4 * 4) = ld4<T>(kb + j * rs + c4 * 4);
            *(f32x4*)(vs + kk * PITCH + c4 * 4) = ld4<T>(vb + j * rs + c4 * 4);
        }
        __syncthreads();
        for (int kk = 0; kk < TK; kk++) {
            float sd = 0.f, pd = 0.f;
#pragma unroll
            for (int d = 0; d < DQ; d++) {
                sd = __builtin_fmaf(q[d], ks[kk * PITCH + part * DQ + d], sd);
                pd = __builtin_fmaf(dq[d], vs[kk * PITCH + part * DQ + d], pd);
            }
            sd = item_sum<LANES>(sd);
            pd = item_sum<LANES>(pd);
            const int j = t0 + kk;
            const bool ok = row_ok && j < j1 && extra_pair(g, i, j);
            const float pe = ok ? fast_exp2(sd * g.scale_log2 - lse2) : 0.f;
            const float ds = pe * (pd - dlt);
#pragma unroll
            for (int d = 0; d < DQ; d++)
                acc[d] = __builtin_fmaf(ds, ks[kk * PITCH + part * DQ + d], acc[d]);
        }
    }
    if (!row_ok) return;
    float* out = g.dq_acc + (((size_t)b * g.Hq + hq) * g.n_global + gi) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d++) atomicAdd(out + d, acc[d]);
}

// ---- cols_dkdv: dk, dv of global keys over E_col -----------------------------
// grid: (b, kv head, tile of kGlobalBwdItems global keys, row chunk); each key
// takes NT / kGlobalBwdItems lanes
template <int D, typename T>
__global__ __launch_bounds__(NT) void cols_dkdv_kernel(const GlobalBwdParams g) {
    constexpr int LANES = NT / kGlobalBwdItems;
    constexpr int DQ = D / LANES;
    constexpr int PITCH = D + 4;
    __shared__ __attribute__((aligned(16))) float qs[TK * PITCH];
    __shared__ __attribute__((aligned(16))) float gs[TK * PITCH];
    __shared__ float rl[3 * TK];   // lse2, delta, row taken (1) or not (0)
    __shared__ int gp[SWA_MAX_GLOBAL];
    const int tid = threadIdx.x, part = tid % LANES;
    int L = blockIdx.x;
    const int chunk = L % g.n_row_chunks;
    L /= g.n_row_chunks;
    const int kt = L % g.key_tiles;
    L /= g.key_tiles;
    const int kvh = L % g.Hkv;
    const int b = L / g.Hkv;
    const int gk = kt * kGlobalBwdItems + tid / LANES;
    const bool key_ok = gk < g.n_global;
    const int j = key_ok ? g.gpos[gk] : 0;
    copy_gpos(g, gp);

    float kx[DQ], vx[DQ], dk[DQ], dv[DQ];
    const size_t ko = (((size_t)b * g.N + j) * g.Hkv + kvh) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
        const f32x4 a = ld4<T>((const T*)g.k + ko + d);
        const f32x4 c = ld4<T>((const T*)g.v + ko + d);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            kx[d + e] = a[e];
            vx[d + e] = c[e];
            dk[d + e] = dv[d + e] = 0.f;
        }
    }
    const int i0 = chunk * g.row_chunk;
    const int i1 = min(g.N, i0 + g.row_chunk);
    for (int h = 0; h < g.group; h++) {
        const int hq = kvh * g.group + h;
        const T* qb = (const T*)g.q + ((size_t)b * g.N * g.Hq + hq) * D;
        const T* ob = (const T*)g.dout + ((size_t)b * g.N * g.Hq + hq) * D;
        const size_t rs = (size_t)g.Hq * D;
        for (int r0 = i0; r0 < i1; r0 += TK) {
            __syncthreads();
            for (int ci = tid; ci < TK * D / 4; ci += NT) {
                const int ri = ci / (D / 4), c4 = ci % (D / 4);
                const int i = min(r0 + ri, i1 - 1);
                *(f32x4*)(qs + ri * PITCH + c4 * 4) = ld4<T>(qb + i * rs + c4 * 4);
                *(f32x4*)(gs + ri * PITCH + c4 * 4) = ld4<T>(ob + i * rs + c4 * 4);
            }
            if (tid < TK) {
                const int i = r0 + tid;
                const int ic = min(i, i1 - 1);
                const size_t li = ((size_t)b * g.Hq + hq) * g.N + ic;
                rl[tid] = g.lse[li] * kLog2eG;
                rl[TK + tid] = g.delta[li];
                rl[2 * TK + tid] = (i < i1 && !is_global(gp, g.n_global, i)) ? 1.f : 0.f;
            }
            __syncthreads();
            for (int ri = 0; ri < TK; ri++) {
                float sd = 0.f, pd = 0.f;
#pragma unroll
                for (int d = 0; d < DQ; d++) {
                    sd = __builtin_fmaf(kx[d], qs[ri * PITCH + part * DQ + d], sd);
                    pd = __builtin_fmaf(vx[d], gs[ri * PITCH + part * DQ + d], pd);
                }
                sd = item_sum<LANES>(sd);
                pd = item_sum<LANES>(pd);
                const int i = r0 + ri;
                const bool ok = key_ok && rl[2 * TK + ri] != 0.f && extra_pair(g, i, j);
                const float pe = ok ? fast_exp2(sd * g.scale_log2 - rl[ri]) : 0.f;
                const float ds = pe * (pd - rl[TK + ri]);
#pragma unroll
                for (int d = 0; d < DQ; d++) {
                    dk[d] = __builtin_fmaf(ds, qs[ri * PITCH + part * DQ + d], dk[d]);
                    dv[d] = __builtin_fmaf(pe, gs[ri * PITCH + part * DQ + d], dv[d]);
                }
            }
        }
    }
    if (!key_ok) return;
    float* out = g.dkv_acc + (((size_t)b * g.Hkv + kvh) * g.n_global + gk) * 2 * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d++) {
        atomicAdd(out + d, dk[d]);
        atomicAdd(out + D + d, dv[d]);
    }
}

// ---- cols_dq: dq of non-global rows over E_col ------------------------------
// grid: (b, hq, 64-row tile); each row adds its term to dq in place
template <int D, typename T>
__global__ __launch_bounds__(NT) void cols_dq_kernel(const GlobalBwdParams g) {
    constexpr int DQ = D / 4;
    constexpr int PITCH = D + 4;
    __shared__ __attribute__((aligned(16))) float ks[TK * PITCH];
    __shared__ __attribute__((aligned(16))) float vs[TK * PITCH];
    __shared__ int jp[TK];
    __shared__ int gp[SWA_MAX_GLOBAL];
    const int tid = threadIdx.x, part = tid & 3;
    int L = blockIdx.x;
    const int rt = L % g.n_row_tiles_all;
    L /= g.n_row_tiles_all;
    const int hq = L % g.Hq;
    const int b = L / g.Hq;
    const int kvh = hq / g.group;
    copy_gpos(g, gp);
    __syncthreads();
    const int i = rt * ITEMS + (tid >> 2);
    const bool row_ok = i < g.N && !is_global(gp, g.n_global, i);
    const int ic = min(i, g.N - 1);

    float q[DQ], dq[DQ], acc[DQ];
    const size_t qo = (((size_t)b * g.N + ic) * g.Hq + hq) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
        const f32x4 a = ld4<T>((const T*)g.q + qo + d);
        const f32x4 o = ld4<T>((const T*)g.dout + qo + d);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            q[d + e] = a[e];
            dq[d + e] = o[e];
            acc[d + e] = 0.f;
        }
    }
    const size_t lrow = ((size_t)b * g.Hq + hq) * g.N + ic;
    const float lse2 = g.lse[lrow] * kLog2eG;
    const float dlt = g.delta[lrow];
    const T* kb = (const T*)g.k + ((size_t)b * g.N * g.Hkv + kvh) * D;
    const T* vb = (const T*)g.v + ((size_t)b * g.N * g.Hkv + kvh) * D;
    const size_t rs = (size_t)g.Hkv * D;

    for (int t0 = 0; t0 < g.n_global; t0 += TK) {
        __syncthreads();
        for (int ci = tid; ci < TK * D / 4; ci += NT) {
            const int kk = ci / (D / 4), c4 = ci % (D / 4);
            const int j = gp[min(t0 + kk, g.n_global - 1)];
            *(f32x4*)(ks + kk * PITCH + c4 * 4) = ld4<T>(kb + j * rs + c4 * 4);
            *(f32x4*)(vs + kk * PITCH + c4 * 4) = ld4<T>(vb + j * rs + c4 * 4);
        }
        if (tid < TK) jp[tid] = t0 + tid < g.n_global ? gp[t0 + tid] : -1;
        __syncthreads();
        for (int kk = 0; kk < TK; kk++) {
            float sd = 0.f, pd = 0.f;
#pragma unroll
            for (int d = 0; d < DQ; d++) {
                sd = __builtin_fmaf(q[d], ks[kk * PITCH + part * DQ + d], sd);
                pd = __builtin_fmaf(dq[d], vs[kk * PITCH + part * DQ + d], pd);
            }
            sd = quad_sum(sd);
            pd = quad_sum(pd);
            const int j = jp[kk];
            const bool ok = row_ok && j >= 0 && extra_pair(g, i, j);
            const float pe = ok ? fast_exp2(sd * g.scale_log2 - lse2) : 0.f;
            const float ds = pe * (pd - dlt);
#pragma unroll
            for (int d = 0; d < DQ; d++)
                acc[d] = __builtin_fmaf(ds, ks[kk * PITCH + part * DQ + d], acc[d]);
        }
    }
    if (!row_ok) return;
    T* out = (T*)g.dq + qo;
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
        f32x4 x = ld4<T>(out + d);
#pragma unroll
        for (int e = 0; e < 4; e++) x[e] += acc[d + e] * g.scale;
        st4<T>(out + d, x);
    }
}

// ---- rows_dkdv: dk, dv of every key over E_row --------------------------------
// grid: (b, kv head, 64-key tile); each key adds its terms to dk, dv in place
template <int D, typename T>
__global__ __launch_bounds__(NT) void rows_dkdv_kernel(const GlobalBwdParams g) {
    constexpr int DQ = D / 4;
    constexpr int PITCH = D + 4;
    __shared__ __attribute__((aligned(16))) float qs[TK * PITCH];
    __shared__ __attribute__((aligned(16))) float gs[TK * PITCH];
    __shared__ float rl[2 * TK];   // lse2, delta
    __shared__ int ip[TK];
    const int tid = threadIdx.x, part = tid & 3;
    int L = blockIdx.x;
    const int kt = L % g.n_key_tiles_all;
    L /= g.n_key_tiles_all;
    const int kvh = L % g.Hkv;
    const int b = L / g.Hkv;
    const int j = kt * ITEMS + (tid >> 2);
    const bool key_ok = j < g.N;
    const int jc = min(j, g.N - 1);

    float kx[DQ], vx[DQ], dk[DQ], dv[DQ];
    const size_t ko = (((size_t)b * g.N + jc) * g.Hkv + kvh) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
        const f32x4 a = ld4<T>((const T*)g.k + ko + d);
        const f32x4 c = ld4<T>((const T*)g.v + ko + d);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            kx[d + e] = a[e];
            vx[d + e] = c[e];
            dk[d + e] = dv[d + e] = 0.f;
        }
    }
    for (int h = 0; h < g.group; h++) {
        const int hq = kvh * g.group + h;
        const T* qb = (const T*)g.q + ((size_t)b * g.N * g.Hq + hq) * D;
        const T* ob = (const T*)g.dout + ((size_t)b * g.N * g.Hq + hq) * D;
        const size_t rs = (size_t)g.Hq * D;
        for (int r0 = 0; r0 < g.n_global; r0 += TK) {
            __syncthreads();
            for (int ci = tid; ci < TK * D / 4; ci += NT) {
                const int ri = ci / (D / 4), c4 = ci % (D / 4);
                const int i = g.gpos[min(r0 + ri, g.n_global - 1)];
                *(f32x4*)(qs + ri * PITCH + c4 * 4) = ld4<T>(qb + i * rs + c4 * 4);
                *(f32x4*)(gs + ri * PITCH + c4 * 4) = ld4<T>(ob + i * rs + c4 * 4);
            }
            if (tid < TK) {
                const bool real = r0 + tid < g.n_global;
                const int i = g.gpos[min(r0 + tid, g.n_global - 1)];
                const size_t li = ((size_t)b * g.Hq + hq) * g.N + i;
                rl[tid] = g.lse[li] * kLog2eG;
                rl[TK + tid] = g.delta[li];
                ip[tid] = real ? i : -1;
            }
            __syncthreads();
            for (int ri = 0; ri < TK; ri++) {
                float sd = 0.f, pd = 0.f;
#pragma unroll
                for (int d = 0; d < DQ; d++) {
                    sd = __builtin_fmaf(kx[d], qs[ri * PITCH + part * DQ + d], sd);
                    pd = __builtin_fmaf(vx[d], gs[ri * PITCH + part * DQ + d], pd);
                }
                sd = quad_sum(sd);
                pd = quad_sum(pd);
                const int i = ip[ri];
                const bool ok = key_ok && i >= 0 && extra_pair(g, i, j);
                const float pe = ok ? fast_exp2(sd * g.scale_log2 - rl[ri]) : 0.f;
                const float ds = pe * (pd - rl[TK + ri]);
#pragma unroll
                for (int d = 0; d < DQ; d++) {
                    dk[d] = __builtin_fmaf(ds, qs[ri * PITCH + part * DQ + d], dk[d]);
                    dv[d] = __builtin_fmaf(pe, gs[ri * PITCH + part * DQ + d], dv[d]);
                }
            }
        }
    }
    if (!key_ok) return;
    T* kp = (T*)g.dk + ko;
    T* vp = (T*)g.dv + ko;
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
        f32x4 x = ld4<T>(kp + d), y = ld4<T>(vp + d);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            x[e] += dk[d + e] * g.scale;
            y[e] += dv[d + e];
        }
        st4<T>(kp + d, x);
        st4<T>(vp + d, y);
    }
}

// ---- accumulators ------------------------------------------------------------------
__global__ __launch_bounds__(NT) void zero_kernel(float* p, size_t n) {
    const size_t i = (size_t)blockIdx.x * NT + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// dq of global rows += scale * dq_acc; one thread per element
template <int D, typename T>
__global__ __launch_bounds__(NT) void add_dq_kernel(const GlobalBwdParams g) {
    const size_t e = (size_t)blockIdx.x * NT + threadIdx.x;
    const size_t total = (size_t)g.B * g.Hq * g.n_global * D;
    if (e >= total) return;
    const int d = (int)(e % D);
    size_t r = e / D;
    const int gi = (int)(r % g.n_global);
    r /= g.n_global;
    const int hq = (int)(r % g.Hq);
    const int b = (int)(r / g.Hq);
    T* p = (T*)g.dq + (((size_t)b * g.N + g.gpos[gi]) * g.Hq + hq) * D + d;
    *p = (T)((float)*p + g.scale * g.dq_acc[e]);
}

// dk, dv of global keys += (scale * dk_acc, dv_acc); one thread per element
template <int D, typename T>
__global__ __launch_bounds__(NT) void add_dkdv_kernel(const GlobalBwdParams g) {
    const size_t e = (size_t)blockIdx.x * NT + threadIdx.x;
    const size_t total = (size_t)g.B * g.Hkv * g.n_global * D;
    if (e >= total) return;
    const int d = (int)(e % D);
    size_t r = e / D;
    const int gk = (int)(r % g.n_global);
    r /= g.n_global;
    const int kvh = (int)(r % g.Hkv);
    const int b = (int)(r / g.Hkv);
    const float* acc = g.dkv_acc + (((size_t)b * g.Hkv + kvh) * g.n_global + gk) * 2 * D;
    const size_t o = (((size_t)b * g.N + g.gpos[gk]) * g.Hkv + kvh) * D + d;
    T* kp = (T*)g.dk + o;
    T* vp = (T*)g.dv + o;
    *kp = (T)((float)*kp + g.scale * acc[d]);
    *vp = (T)((float)*vp + acc[D + d]);
}

unsigned blocks_for(size_t n) { return (unsigned)((n + NT - 1) / NT); }

template <int D, typename T>
hipError_t launch_all(const GlobalBwdParams& g, hipStream_t s) {
    const size_t nq = (size_t)g.B * g.Hq * g.n_global * D;
    const size_t nkv = (size_t)g.B * g.Hkv * g.n_global * 2 * D;
    hipLaunchKernelGGL(zero_kernel, dim3(blocks_for(nq)), dim3(NT), 0, s, g.dq_acc, nq);
    hipLaunchKernelGGL(zero_kernel, dim3(blocks_for(nkv)), dim3(NT), 0, s, g.dkv_acc, nkv);
    hipLaunchKernelGGL((rows_dq_kernel<D, T>),
                       dim3(g.B * g.Hq * g.row_tiles * g.n_key_chunks), dim3(NT), 0, s, g);
    hipLaunchKernelGGL((cols_dkdv_kernel<D, T>),
                       dim3(g.B * g.Hkv * g.key_tiles * g.n_row_chunks), dim3(NT), 0, s, g);
    hipLaunchKernelGGL((cols_dq_kernel<D, T>), dim3(g.B * g.Hq * g.n_row_tiles_all), dim3(NT), 0,
                       s, g);
    hipLaunchKernelGGL((rows_dkdv_kernel<D, T>), dim3(g.B * g.Hkv * g.n_key_tiles_all), dim3(NT),
                       0, s, g);
    hipLaunchKernelGGL((add_dq_kernel<D, T>), dim3(blocks_for(nq)), dim3(NT), 0, s, g);
    hipLaunchKernelGGL((add_dkdv_kernel<D, T>), dim3(blocks_for(nkv / 2)), dim3(NT), 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_global(const GlobalBwdParams& g, int D, int dtype, hipStream_t s) {
    if (dtype == SWA_BF16) return D == 128 ? launch_all<128, __bf16>(g, s) : launch_all<64, __bf16>(g, s);
    return D == 128 ? launch_all<128, float>(g, s) : launch_all<64, float>(g, s);
}

}  // namespace swa
