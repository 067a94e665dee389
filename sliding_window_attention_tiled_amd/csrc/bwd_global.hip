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
// each with j <= i when causal.  Same chain rule as the band passes:
// dS = P (dP - delta), dq = scale sum dS k, dk = scale sum dS q,
// dv = sum P dout.  Four passes:
//   rows_dq    dq of global rows over E_row, one float32 partial per key chunk
//   rows_dkdv  dk, dv of every key over E_row, read-modify-write
//   cols_dq    dq of non-global rows over E_col, read-modify-write
//   cols_dkdv  dk, dv of global keys over E_col, one float32 partial per row chunk
//   add_dq / add_dkdv sum the partials in chunk order into dq / dk, dv
//   (in bf16, rows_dkdv, when launched, sums the cols_dkdv partials of the
//   global keys itself, so that each gradient is rounded once after the band
//   pass, and add_dkdv is not launched).
// In bf16 the band dq pass walks the global keys after its band (cols_dq is
// not launched), and at D = 64 the band dk/dv pass stages the global rows
// after its band (rows_dkdv is not launched): GlobalBwdParams::fused says
// which.  Every sum has a fixed order (no atomics), so the backward is
// bitwise repeatable.
// bf16 runs them on MFMA with the global tokens of a 16-wide block as the
// columns of 16x16 tiles; float32 runs them on the vector ALUs, rows (or keys)
// of a workgroup spread over lanes with tiles of 32 partners staged in LDS.
// The vector passes over all N rows or keys take 64 per workgroup, four lanes
// each; those whose items are the global tokens take kGlobalBwdItems per
// workgroup, sixteen lanes each, so that a few tokens still fill the
// workgroup.
#include <hip/hip_runtime.h>

#include <type_traits>

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

// index of position j in the sorted global list, -1 if j is not global
__device__ __forceinline__ int global_index(const GlobalBwdParams& g, int j) {
    int lo = 0, hi = g.n_global - 1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const int x = g.gpos[mid];
        if (x == j) return mid;
        if (x < j) lo = mid + 1;
        else hi = mid - 1;
    }
    return -1;
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
    float* out = g.dq_part +
                 ((((size_t)b * g.Hq + hq) * g.n_global + gi) * g.n_key_chunks + chunk) * D +
                 part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d++) out[d] = acc[d];
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
    float* out = g.dkv_part +
                 ((((size_t)b * g.Hkv + kvh) * g.n_global + gk) * g.n_row_chunks + chunk) * 2 * D +
                 part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d++) {
        out[d] = dk[d];
        out[D + d] = dv[d];
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

// ---- bf16 passes on MFMA ----------------------------------------------------------
// The global tokens of a 16-wide block are the 16 columns (or rows) of 16x16
// MFMA tiles, the partners (keys or query rows) come 16 per wave step.  Scores
// and dP are 16x16x32 products over D; the second products (dq, dk, dv) are
// 16x16x16 products over the 16 partners or the 16 global tokens, whose
// operand is the score tile's accumulator layout converted to bf16.  The other
// operand of a second product is the transpose of a 16-row block (K, Q or
// dout), read from LDS with ds_read_b64_tr_b16.  Lane roles: l16 = lane % 16
// is the tile column, grp = lane / 16 picks rows 4 grp .. 4 grp + 3 of an
// accumulator and the 8-element slice grp of a 32-deep k-step.
constexpr int kMfmaNT = 256;  // four waves

__device__ __forceinline__ f32x4 mma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i16x4 to_bf16x4(float a, float b, float c, float d) {
    return __builtin_bit_cast(i16x4, bf16x4{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d});
}
// Transposed 16x16 operand of a second product from a row-major block X
// (rows = partners or global tokens, pitch P elements): lane (grp, l16)
// receives X[4 grp + e][16 db + l16] for e = 0..3.
template <int P>
__device__ __forceinline__ i16x4 tr_block(const __bf16* x, int grp, int l16, int db) {
    return lds_read_tr16(x + (grp * 4 + (l16 >> 2)) * P + db * 16 + 4 * (l16 & 3));
}
// the pair is outside the band (and allowed by causality); dilation 1 skips
// the residue test
__device__ __forceinline__ bool extra_pair_fast(const GlobalBwdParams& g, int i, int j) {
    if (g.causal && j > i) return false;
    if (g.dil == 1) {
        const int diff = j - i;
        return diff < -g.wl || diff > g.wr;
    }
    return !in_band(g, i, j);
}

// rows_dq: dq of global rows over E_row.  grid (b, hq, 16 global rows, key
// chunk); waves take 16-key blocks in turn.  S^T = K Q_G^T puts the global rows
// in the columns, so dS^T is the A operand of dq_G = dS K; the wave stages its
// K block in LDS for the transposed B operand.  The four waves' dq_G are summed
// in LDS in wave order and stored as the chunk's float32 partial.
template <int D>
__global__ __launch_bounds__(kMfmaNT) void rows_dq_mfma_kernel(const GlobalBwdParams g) {
    constexpr int KS = D / 32, DB = D / 16, P = D + 8;
    __shared__ __attribute__((aligned(16))) __bf16 kl[4][16 * P];
    __shared__ float red[4][16 * D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    int L = blockIdx.x;
    const int chunk = L % g.n_key_chunks;
    L /= g.n_key_chunks;
    const int rt = L % g.row_tiles;
    L /= g.row_tiles;
    const int hq = L % g.Hq;
    const int b = L / g.Hq;
    const int kvh = hq / g.group;

    const int gi = rt * 16 + l16;
    const bool gi_ok = gi < g.n_global;
    const int irow = gi_ok ? g.gpos[gi] : 0;
    const size_t qo = (((size_t)b * g.N + irow) * g.Hq + hq) * D + grp * 8;
    bf16x8 qb[KS], ob[KS];
#pragma unroll
    for (int k = 0; k < KS; k++) {
        qb[k] = *(const bf16x8*)((const __bf16*)g.q + qo + k * 32);
        ob[k] = *(const bf16x8*)((const __bf16*)g.dout + qo + k * 32);
    }
    const size_t lrow = ((size_t)b * g.Hq + hq) * g.N + irow;
    const float lse2 = g.lse[lrow] * kLog2eG;
    const float dlt = g.delta[lrow];
    f32x4 acc[DB];
#pragma unroll
    for (int d = 0; d < DB; d++) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int j0 = chunk * g.key_chunk;
    const int j1 = min(g.N, j0 + g.key_chunk);
    const size_t rs = (size_t)g.Hkv * D;
    const __bf16* kb = (const __bf16*)g.k + ((size_t)b * g.N * g.Hkv + kvh) * D + grp * 8;
    const __bf16* vb = (const __bf16*)g.v + ((size_t)b * g.N * g.Hkv + kvh) * D + grp * 8;
    __bf16* kw = kl[wave];
    // the next block's K and V rows are loaded while this one is processed
    bf16x8 kn[KS], vn[KS];
    auto load_block = [&](int k0) __attribute__((always_inline)) {
        const size_t jo = (size_t)min(k0 + l16, j1 - 1) * rs;  // masked below
#pragma unroll
        for (int k = 0; k < KS; k++) {
            kn[k] = *(const bf16x8*)(kb + jo + k * 32);
            vn[k] = *(const bf16x8*)(vb + jo + k * 32);
        }
    };
    if (j0 + wave * 16 < j1) load_block(j0 + wave * 16);
    for (int k0 = j0 + wave * 16; k0 < j1; k0 += 64) {
        bf16x8 ka[KS], va[KS];
#pragma unroll
        for (int k = 0; k < KS; k++) {
            ka[k] = kn[k];
            va[k] = vn[k];
        }
        if (k0 + 64 < j1) load_block(k0 + 64);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < KS; k++) *(bf16x8*)(kw + l16 * P + k * 32 + grp * 8) = ka[k];
        __builtin_amdgcn_wave_barrier();
        f32x4 st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; k++) {
            st = mma_k32(ka[k], qb[k], st);
            dpt = mma_k32(va[k], ob[k], dpt);
        }
        // column: global row gi; rows: keys k0 + 4 grp + e
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int j = k0 + grp * 4 + e;
            const bool ok = gi_ok && j < j1 && extra_pair_fast(g, irow, j);
            const float pe = ok ? fast_exp2(st[e] * g.scale_log2 - lse2) : 0.f;
            ds[e] = pe * (dpt[e] - dlt);
        }
        const i16x4 dsa = to_bf16x4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
        for (int d = 0; d < DB; d++) acc[d] = mma_k16(dsa, tr_block<P>(kw, grp, l16, d), acc[d]);
    }
    // acc[d][e]: global row rt*16 + 4 grp + e, dimension 16 d + l16
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
        for (int e = 0; e < 4; e++) red[wave][(grp * 4 + e) * D + d * 16 + l16] = acc[d][e];
    __syncthreads();
    for (int i = threadIdx.x; i < 16 * D; i += kMfmaNT) {
        const int r = rt * 16 + i / D;
        if (r < g.n_global)
            g.dq_part[((((size_t)b * g.Hq + hq) * g.n_global + r) * g.n_key_chunks + chunk) * D +
                      i % D] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
    }
}

// rows_dkdv: dk, dv of every key over E_row.  grid (b, kv head, 64-key tile);
// wave w owns keys 16 w .. 16 w + 15 of the tile.  For each query head of the
// group and each 16-row block of global rows (staged in LDS by the
// workgroup): S = Q_G K^T with the keys in the columns, so dS and P are the B
// operands of dk^T = Q_G^T dS and dv^T = dout_G^T P.  Each key adds its terms
// to dk, dv in place.
template <int D>
__global__ __launch_bounds__(kMfmaNT) void rows_dkdv_mfma_kernel(const GlobalBwdParams g) {
    constexpr int KS = D / 32, DB = D / 16, P = D + 8, CPR = D / 8;
    __shared__ __attribute__((aligned(16))) __bf16 qs[16 * P];
    __shared__ __attribute__((aligned(16))) __bf16 os[16 * P];
    __shared__ float rl[32];  // lse2, delta of the block's rows
    __shared__ int rp[16];    // their positions, -1 past the last global
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    int L = blockIdx.x;
    const int kt = L % g.n_key_tiles_all;
    L /= g.n_key_tiles_all;
    const int kvh = L % g.Hkv;
    const int b = L / g.Hkv;
    const int j = kt * 64 + wave * 16 + l16;
    const bool j_ok = j < g.N;
    const size_t ko = (((size_t)b * g.N + min(j, g.N - 1)) * g.Hkv + kvh) * D;
    bf16x8 kb[KS], vb[KS];
#pragma unroll
    for (int k = 0; k < KS; k++) {
        kb[k] = *(const bf16x8*)((const __bf16*)g.k + ko + k * 32 + grp * 8);
        vb[k] = *(const bf16x8*)((const __bf16*)g.v + ko + k * 32 + grp * 8);
    }
    f32x4 dkt[DB], dvt[DB];
#pragma unroll
    for (int d = 0; d < DB; d++) dkt[d] = dvt[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the band passes' dk, dv of this key (dimensions 16 d + 4 grp + e), read
    // now so that the loads overlap the work below
    __bf16* kp = (__bf16*)g.dk + ko + grp * 4;
    __bf16* vp = (__bf16*)g.dv + ko + grp * 4;
    bf16x4 dk0[DB], dv0[DB];
#pragma unroll
    for (int d = 0; d < DB; d++) {
        dk0[d] = *(const bf16x4*)(kp + d * 16);
        dv0[d] = *(const bf16x4*)(vp + d * 16);
    }

    for (int h = 0; h < g.group; h++) {
        const int hq = kvh * g.group + h;
        for (int rt = 0; rt < g.row_tiles; rt++) {
            __syncthreads();
            for (int ci = tid; ci < 16 * CPR; ci += kMfmaNT) {
                const int r = ci / CPR, c = ci % CPR;
                const int pos = g.gpos[min(rt * 16 + r, g.n_global - 1)];
                const size_t o = (((size_t)b * g.N + pos) * g.Hq + hq) * D + c * 8;
                *(bf16x8*)(qs + r * P + c * 8) = *(const bf16x8*)((const __bf16*)g.q + o);
                *(bf16x8*)(os + r * P + c * 8) = *(const bf16x8*)((const __bf16*)g.dout + o);
            }
            if (tid < 16) {
                const int gi = rt * 16 + tid;
                const int pos = g.gpos[min(gi, g.n_global - 1)];
                const size_t li = ((size_t)b * g.Hq + hq) * g.N + pos;
                rl[tid] = g.lse[li] * kLog2eG;
                rl[16 + tid] = g.delta[li];
                rp[tid] = gi < g.n_global ? pos : -1;
            }
            __syncthreads();
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KS; k++) {
                s = mma_k32(*(const bf16x8*)(qs + l16 * P + k * 32 + grp * 8), kb[k], s);
                dp = mma_k32(*(const bf16x8*)(os + l16 * P + k * 32 + grp * 8), vb[k], dp);
            }
            // column: key j; rows: global rows rt*16 + 4 grp + e
            float pe[4], ds[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = grp * 4 + e;
                const int i = rp[r];
                const bool ok = j_ok && i >= 0 && extra_pair_fast(g, i, j);
                pe[e] = ok ? fast_exp2(s[e] * g.scale_log2 - rl[r]) : 0.f;
                ds[e] = pe[e] * (dp[e] - rl[16 + r]);
            }
            const i16x4 pb = to_bf16x4(pe[0], pe[1], pe[2], pe[3]);
            const i16x4 dsb = to_bf16x4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
            for (int d = 0; d < DB; d++) {
                dkt[d] = mma_k16(tr_block<P>(qs, grp, l16, d), dsb, dkt[d]);
                dvt[d] = mma_k16(tr_block<P>(os, grp, l16, d), pb, dvt[d]);
            }
        }
    }
    if (!j_ok) return;
    // A global key also has pairs with the rows outside its band, which
    // cols_dkdv (launched before this kernel) left as float32 partials.  They
    // are summed here in chunk order, as add_dkdv would, so that the key's
    // gradient is rounded to bf16 once after the band pass, not twice.
    const int gk = global_index(g, j);
    if (gk >= 0) {
        const float* part =
            g.dkv_part + (((size_t)b * g.Hkv + kvh) * g.n_global + gk) * g.n_row_chunks * 2 * D;
#pragma unroll
        for (int d = 0; d < DB; d++) {
            f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < g.n_row_chunks; c++) {
                sk += *(const f32x4*)(part + (size_t)c * 2 * D + d * 16 + grp * 4);
                sv += *(const f32x4*)(part + (size_t)c * 2 * D + D + d * 16 + grp * 4);
            }
            dkt[d] += sk;
            dvt[d] += sv;
        }
    }
    // dkt[d][e]: dimension 16 d + 4 grp + e of key j
#pragma unroll
    for (int d = 0; d < DB; d++) {
        f32x4 x, y;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            x[e] = (float)dk0[d][e] + dkt[d][e] * g.scale;
            y[e] = (float)dv0[d][e] + dvt[d][e];
        }
        st4<__bf16>(kp + d * 16, x);
        st4<__bf16>(vp + d * 16, y);
    }
}

// cols_dq: dq of non-global rows over E_col.  grid (b, hq, 64-row tile); wave
// w owns rows 16 w .. 16 w + 15.  For each 16-key block of global keys (staged
// in LDS by the workgroup): S^T = K_G Q^T with the rows in the columns, so
// dS^T is the B operand of dq^T = K_G^T dS^T.  Each row adds its term to dq in
// place.
template <int D>
__global__ __launch_bounds__(kMfmaNT) void cols_dq_mfma_kernel(const GlobalBwdParams g) {
    constexpr int KS = D / 32, DB = D / 16, P = D + 8, CPR = D / 8;
    __shared__ __attribute__((aligned(16))) __bf16 ks[16 * P];
    __shared__ __attribute__((aligned(16))) __bf16 vs[16 * P];
    __shared__ int gp[SWA_MAX_GLOBAL];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    int L = blockIdx.x;
    const int rt = L % g.n_row_tiles_all;
    L /= g.n_row_tiles_all;
    const int hq = L % g.Hq;
    const int b = L / g.Hq;
    const int kvh = hq / g.group;
    for (int i = tid; i < g.n_global; i += kMfmaNT) gp[i] = g.gpos[i];
    __syncthreads();
    const int i = rt * 64 + wave * 16 + l16;
    const bool row_ok = i < g.N && !is_global(gp, g.n_global, i);
    const int ic = min(i, g.N - 1);
    const size_t qo = (((size_t)b * g.N + ic) * g.Hq + hq) * D;
    bf16x8 qb[KS], ob[KS];
#pragma unroll
    for (int k = 0; k < KS; k++) {
        qb[k] = *(const bf16x8*)((const __bf16*)g.q + qo + k * 32 + grp * 8);
        ob[k] = *(const bf16x8*)((const __bf16*)g.dout + qo + k * 32 + grp * 8);
    }
    const size_t lrow = ((size_t)b * g.Hq + hq) * g.N + ic;
    const float lse2 = g.lse[lrow] * kLog2eG;
    const float dlt = g.delta[lrow];
    f32x4 dqt[DB];
#pragma unroll
    for (int d = 0; d < DB; d++) dqt[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the band passes' dq of this row (dimensions 16 d + 4 grp + e), read now
    // so that the loads overlap the work below
    __bf16* qp = (__bf16*)g.dq + qo + grp * 4;
    bf16x4 dq0[DB];
#pragma unroll
    for (int d = 0; d < DB; d++) dq0[d] = *(const bf16x4*)(qp + d * 16);

    for (int kt = 0; kt < g.key_tiles; kt++) {
        __syncthreads();
        for (int ci = tid; ci < 16 * CPR; ci += kMfmaNT) {
            const int r = ci / CPR, c = ci % CPR;
            const int pos = gp[min(kt * 16 + r, g.n_global - 1)];
            const size_t o = (((size_t)b * g.N + pos) * g.Hkv + kvh) * D + c * 8;
            *(bf16x8*)(ks + r * P + c * 8) = *(const bf16x8*)((const __bf16*)g.k + o);
            *(bf16x8*)(vs + r * P + c * 8) = *(const bf16x8*)((const __bf16*)g.v + o);
        }
        __syncthreads();
        f32x4 st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; k++) {
            st = mma_k32(*(const bf16x8*)(ks + l16 * P + k * 32 + grp * 8), qb[k], st);
            dpt = mma_k32(*(const bf16x8*)(vs + l16 * P + k * 32 + grp * 8), ob[k], dpt);
        }
        // column: row i; rows: global keys kt*16 + 4 grp + e
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int gk = kt * 16 + grp * 4 + e;
            const bool ok = row_ok && gk < g.n_global && extra_pair_fast(g, i, gp[gk]);
            const float pe = ok ? fast_exp2(st[e] * g.scale_log2 - lse2) : 0.f;
            ds[e] = pe * (dpt[e] - dlt);
        }
        const i16x4 dsb = to_bf16x4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
        for (int d = 0; d < DB; d++) dqt[d] = mma_k16(tr_block<P>(ks, grp, l16, d), dsb, dqt[d]);
    }
    if (!row_ok) return;
    // dqt[d][e]: dimension 16 d + 4 grp + e of row i
#pragma unroll
    for (int d = 0; d < DB; d++) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; e++) x[e] = (float)dq0[d][e] + dqt[d][e] * g.scale;
        st4<__bf16>(qp + d * 16, x);
    }
}

// cols_dkdv: dk, dv of global keys over E_col.  grid (b, kv head, 16 global
// keys, row chunk); waves take 16-row blocks in turn, for every query head of
// the group.  S = Q K_G^T puts the global keys in the columns, so dS^T and P^T
// are the A operands of dk_G = dS^T Q and dv_G = P^T dout; the wave stages its
// Q and dout blocks in LDS for the transposed B operands.  The four waves'
// sums are added in LDS in wave order and stored as the chunk's float32
// partial.
template <int D>
__global__ __launch_bounds__(kMfmaNT) void cols_dkdv_mfma_kernel(const GlobalBwdParams g) {
    constexpr int KS = D / 32, DB = D / 16, P = D + 8;
    __shared__ __attribute__((aligned(16))) __bf16 qw[4][16 * P];
    __shared__ __attribute__((aligned(16))) __bf16 ow[4][16 * P];
    __shared__ float red[4][16 * 2 * D];
    __shared__ int gp[SWA_MAX_GLOBAL];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    int L = blockIdx.x;
    const int chunk = L % g.n_row_chunks;
    L /= g.n_row_chunks;
    const int kt = L % g.key_tiles;
    L /= g.key_tiles;
    const int kvh = L % g.Hkv;
    const int b = L / g.Hkv;
    for (int i = tid; i < g.n_global; i += kMfmaNT) gp[i] = g.gpos[i];
    __syncthreads();
    const int gk = kt * 16 + l16;
    const bool gk_ok = gk < g.n_global;
    const int jpos = gp[min(gk, g.n_global - 1)];
    const size_t ko = (((size_t)b * g.N + jpos) * g.Hkv + kvh) * D + grp * 8;
    bf16x8 kb[KS], vb[KS];
#pragma unroll
    for (int k = 0; k < KS; k++) {
        kb[k] = *(const bf16x8*)((const __bf16*)g.k + ko + k * 32);
        vb[k] = *(const bf16x8*)((const __bf16*)g.v + ko + k * 32);
    }
    f32x4 dkg[DB], dvg[DB];
#pragma unroll
    for (int d = 0; d < DB; d++) dkg[d] = dvg[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int i0 = chunk * g.row_chunk;
    const int i1 = min(g.N, i0 + g.row_chunk);
    __bf16* qx = qw[wave];
    __bf16* ox = ow[wave];
    for (int h = 0; h < g.group; h++) {
        const int hq = kvh * g.group + h;
        const size_t rs = (size_t)g.Hq * D;
        const __bf16* qh = (const __bf16*)g.q + ((size_t)b * g.N * g.Hq + hq) * D + grp * 8;
        const __bf16* oh = (const __bf16*)g.dout + ((size_t)b * g.N * g.Hq + hq) * D + grp * 8;
        const float* lh = g.lse + ((size_t)b * g.Hq + hq) * g.N;
        const float* dh = g.delta + ((size_t)b * g.Hq + hq) * g.N;
        // the next block's Q and dout rows are loaded while this one is processed
        bf16x8 qn[KS], on[KS];
        auto load_block = [&](const __bf16* qs_, const __bf16* os_, int r0)
                              __attribute__((always_inline)) {
            const size_t ro = (size_t)min(r0 + l16, i1 - 1) * rs;  // masked below
#pragma unroll
            for (int k = 0; k < KS; k++) {
                qn[k] = *(const bf16x8*)(qs_ + ro + k * 32);
                on[k] = *(const bf16x8*)(os_ + ro + k * 32);
            }
        };
        if (i0 + wave * 16 < i1) load_block(qh, oh, i0 + wave * 16);
        int cur = 0;  // first global position >= r0 (the wave's blocks ascend)
        for (int r0 = i0 + wave * 16; r0 < i1; r0 += 64) {
            // bit r of gmask: row r0 + r is a global row
            while (cur < g.n_global && gp[cur] < r0) cur++;
            unsigned gmask = 0;
            if (cur + l16 < g.n_global && gp[cur + l16] < r0 + 16) gmask = 1u << (gp[cur + l16] - r0);
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) gmask |= __shfl_xor(gmask, m);
            bf16x8 qa[KS], oa[KS];
#pragma unroll
            for (int k = 0; k < KS; k++) {
                qa[k] = qn[k];
                oa[k] = on[k];
            }
            if (r0 + 64 < i1) load_block(qh, oh, r0 + 64);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < KS; k++) {
                *(bf16x8*)(qx + l16 * P + k * 32 + grp * 8) = qa[k];
                *(bf16x8*)(ox + l16 * P + k * 32 + grp * 8) = oa[k];
            }
            __builtin_amdgcn_wave_barrier();
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KS; k++) {
                s = mma_k32(qa[k], kb[k], s);
                dp = mma_k32(oa[k], vb[k], dp);
            }
            // column: global key gk; rows: query rows r0 + 4 grp + e
            float pe[4], ds[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int i = r0 + grp * 4 + e;
                const int ic = min(i, i1 - 1);
                const bool ok = gk_ok && i < i1 && !((gmask >> (grp * 4 + e)) & 1u) &&
                                extra_pair_fast(g, i, jpos);
                pe[e] = ok ? fast_exp2(s[e] * g.scale_log2 - lh[ic] * kLog2eG) : 0.f;
                ds[e] = pe[e] * (dp[e] - dh[ic]);
            }
            const i16x4 pa = to_bf16x4(pe[0], pe[1], pe[2], pe[3]);
            const i16x4 dsa = to_bf16x4(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
            for (int d = 0; d < DB; d++) {
                dkg[d] = mma_k16(dsa, tr_block<P>(qx, grp, l16, d), dkg[d]);
                dvg[d] = mma_k16(pa, tr_block<P>(ox, grp, l16, d), dvg[d]);
            }
        }
    }
    // dkg[d][e]: global key kt*16 + 4 grp + e, dimension 16 d + l16
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            red[wave][(grp * 4 + e) * 2 * D + d * 16 + l16] = dkg[d][e];
            red[wave][(grp * 4 + e) * 2 * D + D + d * 16 + l16] = dvg[d][e];
        }
    __syncthreads();
    for (int i = tid; i < 16 * 2 * D; i += kMfmaNT) {
        const int r = kt * 16 + i / (2 * D);
        if (r < g.n_global)
            g.dkv_part[((((size_t)b * g.Hkv + kvh) * g.n_global + r) * g.n_row_chunks + chunk) *
                           2 * D +
                       i % (2 * D)] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
    }
}

// ---- partials ----------------------------------------------------------------------
// dq of global rows += scale * (sum of the key chunks' partials, in chunk
// order); one thread per element
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
    const float* part = g.dq_part + (e / D) * g.n_key_chunks * D + d;
    float sum = 0.f;
    for (int c = 0; c < g.n_key_chunks; c++) sum += part[(size_t)c * D];
    T* p = (T*)g.dq + (((size_t)b * g.N + g.gpos[gi]) * g.Hq + hq) * D + d;
    *p = (T)((float)*p + g.scale * sum);
}

// dk, dv of global keys += (scale * dk, dv summed over the row chunks'
// partials in chunk order); one thread per element
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
    const float* part = g.dkv_part + (e / D) * g.n_row_chunks * 2 * D;
    float sk = 0.f, sv = 0.f;
    for (int c = 0; c < g.n_row_chunks; c++) {
        sk += part[(size_t)c * 2 * D + d];
        sv += part[(size_t)c * 2 * D + D + d];
    }
    const size_t o = (((size_t)b * g.N + g.gpos[gk]) * g.Hkv + kvh) * D + d;
    T* kp = (T*)g.dk + o;
    T* vp = (T*)g.dv + o;
    *kp = (T)((float)*kp + g.scale * sk);
    *vp = (T)((float)*vp + sv);
}

unsigned blocks_for(size_t n) { return (unsigned)((n + NT - 1) / NT); }

template <int D, typename T>
hipError_t launch_all(const GlobalBwdParams& g, hipStream_t s) {
    const size_t nq = (size_t)g.B * g.Hq * g.n_global * D;
    const size_t nkv = (size_t)g.B * g.Hkv * g.n_global * 2 * D;
    const dim3 rows_dq_grid(g.B * g.Hq * g.row_tiles * g.n_key_chunks);
    const dim3 cols_dkdv_grid(g.B * g.Hkv * g.key_tiles * g.n_row_chunks);
    const dim3 cols_dq_grid(g.B * g.Hq * g.n_row_tiles_all);
    const dim3 rows_dkdv_grid(g.B * g.Hkv * g.n_key_tiles_all);
    if constexpr (std::is_same_v<T, __bf16>) {
        hipLaunchKernelGGL((rows_dq_mfma_kernel<D>), rows_dq_grid, dim3(kMfmaNT), 0, s, g);
        hipLaunchKernelGGL((cols_dkdv_mfma_kernel<D>), cols_dkdv_grid, dim3(kMfmaNT), 0, s, g);
        if (!(g.fused & kGlobalColsDqFused))
            hipLaunchKernelGGL((cols_dq_mfma_kernel<D>), cols_dq_grid, dim3(kMfmaNT), 0, s, g);
        if (!(g.fused & kGlobalRowsDkdvFused))
            hipLaunchKernelGGL((rows_dkdv_mfma_kernel<D>), rows_dkdv_grid, dim3(kMfmaNT), 0, s, g);
    } else {
        hipLaunchKernelGGL((rows_dq_kernel<D, T>), rows_dq_grid, dim3(NT), 0, s, g);
        hipLaunchKernelGGL((cols_dkdv_kernel<D, T>), cols_dkdv_grid, dim3(NT), 0, s, g);
        hipLaunchKernelGGL((cols_dq_kernel<D, T>), cols_dq_grid, dim3(NT), 0, s, g);
        hipLaunchKernelGGL((rows_dkdv_kernel<D, T>), rows_dkdv_grid, dim3(NT), 0, s, g);
    }
    hipLaunchKernelGGL((add_dq_kernel<D, T>), dim3(blocks_for(nq)), dim3(NT), 0, s, g);
    // bf16 rows_dkdv adds the global keys' partials itself
    const bool dkdv_added = std::is_same_v<T, __bf16> && !(g.fused & kGlobalRowsDkdvFused);
    if (!dkdv_added)
        hipLaunchKernelGGL((add_dkdv_kernel<D, T>), dim3(blocks_for(nkv / 2)), dim3(NT), 0, s, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_global(const GlobalBwdParams& g, int D, int dtype, hipStream_t s) {
    if (dtype == SWA_BF16) return D == 128 ? launch_all<128, __bf16>(g, s) : launch_all<64, __bf16>(g, s);
    return D == 128 ? launch_all<128, float>(g, s) : launch_all<64, float>(g, s);
}

}  // namespace swa
