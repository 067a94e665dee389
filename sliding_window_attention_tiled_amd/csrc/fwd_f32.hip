// fwd_f32.hip -- sliding-window attention forward for float32 inputs.
//
// Same work decomposition and key streams as the bf16 kernel (band tiles of
// one residue class, then gathered global-key tiles; GROWS mode for global
// query rows), evaluated in float32 on the vector ALUs: float32 MFMA would
// add nothing for the sizes this path serves and the vector form keeps every
// product exact to float32 rounding.  A workgroup holds 64 query rows of one
// head, four lanes per row (each a quarter of the head dimension); K/V tiles
// of 32 keys are staged in LDS and the softmax is kept online.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fwd_common.h"
#include "swa_kernels.h"

namespace swa {
namespace {

constexpr int TK = 32;          // keys per tile
constexpr int ROWS = 64;        // query rows per workgroup
constexpr int NT = 256;

template <int D, bool GROWS>
__global__ __launch_bounds__(NT) void swa_fwd_f32_kernel(const FwdParams p) {
    constexpr int DQ = D / 4;   // dims per lane
    constexpr int PITCH = D + 4;
    __shared__ __attribute__((aligned(16))) float ks_lds[TK * PITCH];
    __shared__ __attribute__((aligned(16))) float vs_lds[TK * PITCH];

    const int tid = threadIdx.x;
    const int row_in_wg = tid >> 2;
    const int part = tid & 3;

    const WorkItem wi = GROWS ? decode_grows_item(p, blockIdx.x, ROWS, TK)
                              : decode_band_item(p, xcd_contiguous(blockIdx.x, gridDim.x), TK);
    const KeyStream& ks = wi.ks;
    const int b = wi.b, kvh = wi.kvh;
    const int hq = kvh * p.group + wi.hg;  // one head per workgroup (hpw == 1)

    const int row = wi.row0 + row_in_wg;
    int qpos, qres;
    if (!GROWS) {
        qres = row;
        qpos = row < ks.Nr ? ks.r + row * ks.dil : -1;
    } else {
        qres = 0;
        qpos = row < p.n_global ? p.gpos[row] : -1;
    }
    float q[DQ];
    {
        const float* qp =
            (const float*)p.q + (((size_t)b * p.N + max(qpos, 0)) * p.Hq + hq) * D + part * DQ;
#pragma unroll
        for (int d = 0; d < DQ; d++) q[d] = qpos >= 0 ? qp[d] : 0.f;
    }
    float acc[DQ];
#pragma unroll
    for (int d = 0; d < DQ; d++) acc[d] = 0.f;
    float m_run = kEmptyMax, l_run = 0.f;
    const float c = p.scale_log2;

    const int rowstride = p.Hkv * D;
    const float* kbase = (const float*)p.k + ((size_t)b * p.N * p.Hkv + kvh) * D;
    const float* vbase = (const float*)p.v + ((size_t)b * p.N * p.Hkv + kvh) * D;
    // ring rows of this (b, kv head) for chunked prefill (unused otherwise)
    const size_t ring_off = ((size_t)b * p.Hkv + kvh) * (size_t)p.W * D;
    const float* krbase = (const float*)p.kring + ring_off;
    const float* vrbase = (const float*)p.vring + ring_off;

    for (int j = 0; j < ks.n_tiles; j++) {
        __syncthreads();  // previous tile fully consumed
        for (int ci = tid; ci < TK * D / 4; ci += NT) {
            const int key = ci / (D / 4), c4 = ci % (D / 4);
            const float* ksrc = nullptr;
            const float* vsrc = nullptr;
            const int kk = ks.k_lo + j * TK + key;
            if (!GROWS && j < ks.n_band_tiles && kk < 0) {
                // ring entry (chunked prefill)
                const size_t o = (size_t)ring_slot(ks, kk, p.W) * D + c4 * 4;
                ksrc = krbase + o;
                vsrc = vrbase + o;
            } else {
                const int pos = key_position(ks, p, j, key, TK, GROWS);
                if (pos >= 0) {
                    const size_t o = (size_t)pos * rowstride + c4 * 4;
                    ksrc = kbase + o;
                    vsrc = vbase + o;
                }
            }
            f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
            if (ksrc != nullptr) {
                kv = *(const f32x4*)ksrc;
                vv = *(const f32x4*)vsrc;
            }
            *(f32x4*)(ks_lds + key * PITCH + c4 * 4) = kv;
            *(f32x4*)(vs_lds + key * PITCH + c4 * 4) = vv;
        }
        __syncthreads();

        const bool band_tile = GROWS || j < ks.n_band_tiles;
        float s[TK];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < TK; k++) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < DQ; d++) dot = __builtin_fmaf(q[d], ks_lds[k * PITCH + part * DQ + d], dot);
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            bool valid;
            if (GROWS) {
                const int kk = ks.k_lo + j * TK + k;
                valid = kk <= ks.k_hi && qpos >= 0 && (!p.causal || kk <= qpos);
            } else if (band_tile) {
                const int kk = ks.k_lo + j * TK + k;
                const int dl = kk - qres;
                valid = kk <= ks.k_hi && dl >= -p.wl && dl <= p.wr;
            } else {
                const int gi = (j - ks.n_band_tiles) * TK + k;
                valid = gi < ks.n_global && qpos >= 0 &&
                        global_key_visible(p, ks, p.gpos[gi], qres, qpos);
            }
            s[k] = valid ? dot : -INFINITY;
            mx = fmaxf(mx, s[k]);
        }
        mx *= c;
        const bool up = mx > m_run + kLazyRescale;
        const float m_use = up ? mx : m_run;
        if (up) {
            const float alpha = fast_exp2(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < DQ; d++) acc[d] *= alpha;
        }
        m_run = m_use;
#pragma unroll
        for (int k = 0; k < TK; k++) {
            const float pk = fast_exp2(__builtin_fmaf(s[k], c, -m_use));
            l_run += pk;
#pragma unroll
            for (int d = 0; d < DQ; d++)
                acc[d] = __builtin_fmaf(pk, vs_lds[k * PITCH + part * DQ + d], acc[d]);
        }
    }

    if (qpos < 0) return;
    if (!GROWS) {
        const float inv = 1.0f / l_run;
        float* op = (float*)p.out + (((size_t)b * p.N + qpos) * p.Hq + hq) * D + part * DQ;
#pragma unroll
        for (int d = 0; d < DQ; d++) op[d] = acc[d] * inv;
        if (p.lse != nullptr && part == 0)
            p.lse[((size_t)b * p.Hq + hq) * p.N + qpos] =
                (m_run + __builtin_amdgcn_logf(l_run)) * kLn2;
    } else {
        float* rec = p.partials +
                     ((((size_t)b * p.Hq + hq) * p.n_global + row) * p.g_nchunks + wi.chunk) *
                         (D + kPartialPad);
#pragma unroll
        for (int d = 0; d < DQ; d++) rec[part * DQ + d] = acc[d];
        if (part == 0) {
            rec[D] = m_run;
            rec[D + 1] = l_run;
        }
    }
}

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL((swa_fwd_f32_kernel<D, false>), dim3(p.n_blocks), dim3(NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_global == 0) return e;
    const int grid = p.B * p.Hkv * p.head_groups * p.g_rowgroups * p.g_nchunks;
    hipLaunchKernelGGL((swa_fwd_f32_kernel<D, true>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

}  // namespace

FwdShape fwd_f32_shape(int group) {
    (void)group;
    return FwdShape{1, ROWS, ROWS};
}

hipError_t launch_fwd_f32(const FwdParams& p, int D, hipStream_t s) {
    if (D == 128) return launch_d<128>(p, s);
    return launch_d<64>(p, s);
}

}  // namespace swa
