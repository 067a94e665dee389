// bwd_f32.hip -- backward of the sliding-window attention forward for float32
// inputs, on the vector ALUs (the float32 path serves small problems; every
// product stays exact to float32 rounding).
//
// Same gradients and decomposition as the bf16 backward (chain rule through
// s = scale q.k, the softmax over the attended set and the weighted sum:
// bmjup.com "Sliding window attention", Q&A on training vs inference):
//   query-major: per query row, over the forward's key tiles,
//     dq_i = scale sum_j P_ij (dP_ij - delta_i) k_j;
//   key-major: per key, over the query rows whose windows reach it (every
//     query head of the kv head's group),
//     dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i.
// P is rebuilt from the forward's lse; delta_i = dout_i . out_i comes from the
// delta kernel in bwd_bf16.hip (its float32 instance).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fwd_common.h"
#include "swa_kernels.h"

namespace swa {
namespace {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr int TK = 32;     // keys (or queries) per LDS tile
constexpr int ROWS = 64;   // query rows (or keys) per workgroup
constexpr int NT = 256;    // four lanes per row

template <int D>
__global__ __launch_bounds__(NT) void bwd_dq_f32_kernel(const BwdParams bp) {
    const FwdParams& p = bp.f;
    constexpr int DQ = D / 4;
    constexpr int PITCH = D + 4;
    __shared__ __attribute__((aligned(16))) float ks_lds[TK * PITCH];
    __shared__ __attribute__((aligned(16))) float vs_lds[TK * PITCH];
    const int tid = threadIdx.x;
    const int part = tid & 3;
    const WorkItem wi = decode_band_item(p, xcd_contiguous(blockIdx.x, gridDim.x), TK);
    const KeyStream& ks = wi.ks;
    const int b = wi.b, kvh = wi.kvh;
    const int hq = kvh * p.group + wi.hg;
    const int row = wi.row0 + (tid >> 2);
    const int qres = row;
    const int qpos = row < ks.Nr ? ks.r + row * ks.dil : -1;

    float q[DQ], g[DQ], acc[DQ];
    const size_t qo = (((size_t)b * p.N + max(qpos, 0)) * p.Hq + hq) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d++) {
        q[d] = qpos >= 0 ? ((const float*)p.q)[qo + d] : 0.f;
        g[d] = qpos >= 0 ? ((const float*)bp.dout)[qo + d] : 0.f;
        acc[d] = 0.f;
    }
    const size_t lrow = ((size_t)b * p.Hq + hq) * p.N + max(qpos, 0);
    const float lse2 = qpos >= 0 ? p.lse[lrow] * kLog2eF : 0.f;
    const float dlt = qpos >= 0 ? bp.delta[lrow] : 0.f;
    const float c = p.scale_log2;
    const int rowstride = p.Hkv * D;
    const float* kbase = (const float*)p.k + ((size_t)b * p.N * p.Hkv + kvh) * D;
    const float* vbase = (const float*)p.v + ((size_t)b * p.N * p.Hkv + kvh) * D;

    for (int j = 0; j < ks.n_band_tiles; j++) {
        __syncthreads();
        for (int ci = tid; ci < TK * D / 4; ci += NT) {
            const int key = ci / (D / 4), c4 = ci % (D / 4);
            const int pos = key_position(ks, p, j, key, TK, false);
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (pos >= 0) {
                kv = *(const f32x4*)(kbase + (size_t)pos * rowstride + c4 * 4);
                vv = *(const f32x4*)(vbase + (size_t)pos * rowstride + c4 * 4);
            }
            *(f32x4*)(ks_lds + key * PITCH + c4 * 4) = kv;
            *(f32x4*)(vs_lds + key * PITCH + c4 * 4) = vv;
        }
        __syncthreads();
        for (int k = 0; k < TK; k++) {
            float sd = 0.f, pd = 0.f;
#pragma unroll
            for (int d = 0; d < DQ; d++) {
                sd = __builtin_fmaf(q[d], ks_lds[k * PITCH + part * DQ + d], sd);
                pd = __builtin_fmaf(g[d], vs_lds[k * PITCH + part * DQ + d], pd);
            }
            sd += __shfl_xor(sd, 1);
            sd += __shfl_xor(sd, 2);
            pd += __shfl_xor(pd, 1);
            pd += __shfl_xor(pd, 2);
            const int kk = ks.k_lo + j * TK + k;
            const int dl = kk - qres;
            const bool valid = qpos >= 0 && kk <= ks.k_hi && dl >= -p.wl && dl <= p.wr;
            const float pe = valid ? fast_exp2(sd * c - lse2) : 0.f;
            const float ds = pe * (pd - dlt);
#pragma unroll
            for (int d = 0; d < DQ; d++)
                acc[d] = __builtin_fmaf(ds, ks_lds[k * PITCH + part * DQ + d], acc[d]);
        }
    }
    if (qpos < 0) return;
    float* op = (float*)bp.dq + qo;
#pragma unroll
    for (int d = 0; d < DQ; d++) op[d] = acc[d] * bp.scale;
}

template <int D>
__global__ __launch_bounds__(NT) void bwd_dkdv_f32_kernel(const BwdParams bp) {
    const FwdParams& p = bp.f;
    constexpr int DQ = D / 4;
    constexpr int PITCH = D + 4;
    __shared__ __attribute__((aligned(16))) float qs_lds[TK * PITCH];
    __shared__ __attribute__((aligned(16))) float gs_lds[TK * PITCH];
    __shared__ float rs_lds[2 * TK];
    const int tid = threadIdx.x;
    const int part = tid & 3;

    // longest key blocks first: from the first to the last when the window
    // reaches further left than right (the last blocks' query rows run off the
    // end of the sequence then), else from the last to the first
    const int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int Ls = L % bp.ktiles_per_slab;
    int t = p.wl > p.wr ? Ls : bp.ktiles_per_slab - 1 - Ls;
    const int slab = L / bp.ktiles_per_slab;
    const int kvh = slab % p.Hkv;
    const int b = slab / p.Hkv;
    int r, kt, Nr;
    const int long_total = p.rem * bp.ktiles_long;
    if (t < long_total) {
        r = t / bp.ktiles_long;
        kt = t % bp.ktiles_long;
        Nr = p.qd + 1;
    } else {
        t -= long_total;
        r = p.rem + t / bp.ktiles_short;
        kt = t % bp.ktiles_short;
        Nr = p.qd;
    }
    const int kb0 = kt * ROWS;
    const int kb1 = min(kb0 + ROWS - 1, Nr - 1);
    const int key = kb0 + (tid >> 2);
    const bool key_ok = key <= kb1;
    const int kpos = r + min(key, kb1) * p.dil;
    const int q_lo = max(0, kb0 - p.wr);
    const int q_hi = min(Nr - 1, kb1 + p.wl);
    const int n_qt = (q_hi - q_lo + TK) / TK;

    float k[DQ], v[DQ], dk[DQ], dv[DQ];
    const size_t ko = (((size_t)b * p.N + kpos) * p.Hkv + kvh) * D + part * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d++) {
        k[d] = ((const float*)p.k)[ko + d];
        v[d] = ((const float*)p.v)[ko + d];
        dk[d] = dv[d] = 0.f;
    }
    const float c = p.scale_log2;
    for (int h = 0; h < p.group; h++) {
        const int hq = kvh * p.group + h;
        for (int qt = 0; qt < n_qt; qt++) {
            const int q0 = q_lo + qt * TK;
            __syncthreads();
            for (int ci = tid; ci < TK * D / 4; ci += NT) {
                const int qr = ci / (D / 4), c4 = ci % (D / 4);
                const int qrow = q0 + qr;
                f32x4 qv = {0.f, 0.f, 0.f, 0.f}, gv = {0.f, 0.f, 0.f, 0.f};
                if (qrow <= q_hi) {
                    const size_t off =
                        (((size_t)b * p.N + r + (size_t)qrow * p.dil) * p.Hq + hq) * D + c4 * 4;
                    qv = *(const f32x4*)((const float*)p.q + off);
                    gv = *(const f32x4*)((const float*)bp.dout + off);
                }
                *(f32x4*)(qs_lds + qr * PITCH + c4 * 4) = qv;
                *(f32x4*)(gs_lds + qr * PITCH + c4 * 4) = gv;
            }
            if (tid < 2 * TK) {
                const int qrow = q0 + (tid & (TK - 1));
                float x = 0.f;
                if (qrow <= q_hi) {
                    const size_t li = ((size_t)b * p.Hq + hq) * p.N + r + (size_t)qrow * p.dil;
                    x = tid < TK ? p.lse[li] * kLog2eF : bp.delta[li];
                }
                rs_lds[tid] = x;
            }
            __syncthreads();
            for (int qi = 0; qi < TK; qi++) {
                float sd = 0.f, pd = 0.f;
#pragma unroll
                for (int d = 0; d < DQ; d++) {
                    sd = __builtin_fmaf(k[d], qs_lds[qi * PITCH + part * DQ + d], sd);
                    pd = __builtin_fmaf(v[d], gs_lds[qi * PITCH + part * DQ + d], pd);
                }
                sd += __shfl_xor(sd, 1);
                sd += __shfl_xor(sd, 2);
                pd += __shfl_xor(pd, 1);
                pd += __shfl_xor(pd, 2);
                const int qrow = q0 + qi;
                const int x = qrow - key + p.wr;  // valid when 0 <= x <= wl + wr
                const bool valid = key_ok && qrow <= q_hi && x >= 0 && x <= p.wl + p.wr;
                const float pe = valid ? fast_exp2(sd * c - rs_lds[qi]) : 0.f;
                const float ds = pe * (pd - rs_lds[TK + qi]);
#pragma unroll
                for (int d = 0; d < DQ; d++) {
                    dk[d] = __builtin_fmaf(ds, qs_lds[qi * PITCH + part * DQ + d], dk[d]);
                    dv[d] = __builtin_fmaf(pe, gs_lds[qi * PITCH + part * DQ + d], dv[d]);
                }
            }
        }
    }
    if (!key_ok) return;
#pragma unroll
    for (int d = 0; d < DQ; d++) {
        ((float*)bp.dk)[ko + d] = dk[d] * bp.scale;
        ((float*)bp.dv)[ko + d] = dv[d];
    }
}

template <int D>
hipError_t launch_d(const BwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), dim3(p.f.n_blocks), dim3(NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), dim3(p.k_blocks), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace

FwdShape bwd_f32_dq_shape(int group) {
    (void)group;
    return FwdShape{1, ROWS, ROWS};
}

int bwd_f32_dkdv_keys() { return ROWS; }

hipError_t launch_bwd_f32(const BwdParams& p, int D, hipStream_t s) {
    return D == 128 ? launch_d<128>(p, s) : launch_d<64>(p, s);
}

}  // namespace swa
