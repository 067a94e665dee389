// fwd_f32.hip -- sliding-window attention forward for float32 inputs, on the
// float32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Same work decomposition and key streams as the bf16 kernel (band tiles of
// one residue class, then gathered global-key tiles; GROWS mode for global
// query rows, a partial per key chunk).  A workgroup holds 64 query rows of
// one head, two waves of 32; K/V tiles of 32 keys are staged in LDS.
//
// Scores are formed transposed, S^T = K Q^T, so that each lane holds 16 keys
// of one query row and the row reductions are in-lane plus one exchange with
// lane ^ 32.  One MFMA step contracts two head dimensions; lane half h of
// step 4g + i supplies dimension 8g + 4h + i, for K (A operand, read as one
// 16-byte LDS load per four steps) and Q (B operand, held in registers) alike.
// The weights stay in float32 (no rounding before P V) and the row sum adds
// exactly those.  O^T += V^T P^T contracts two keys per step: the step pairs
// keys 8g + j and 8g + 4 + j, the ones lane halves 0 and 1 hold at element
// 4g + j of their scores, so the B operand is a lane's own weight and V is
// read one float per lane.  The softmax is kept online, with the max moved
// only when a tile exceeds it by more than 2^8 (exact up to rounding).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fwd_common.h"
#include "swa_kernels.h"

namespace swa {
namespace {

constexpr int TK = 32;          // keys per tile
constexpr int NW = 2;           // waves per workgroup, 32 query rows each
constexpr int ROWS = 32 * NW;   // query rows per workgroup
constexpr int NT = 64 * NW;

template <int D, bool GROWS>
__global__ __launch_bounds__(NT) void swa_fwd_f32_kernel(const FwdParams p) {
    constexpr int G = D / 8;     // groups of four MFMA steps (eight dimensions each)
    constexpr int DB = D / 32;   // 32-row blocks of O^T
    // Row pitches (floats).  A K read (16 bytes per lane, 16 lanes per LDS
    // cycle, 16 consecutive rows at one offset) needs rows 4 (mod 64) dwords
    // apart; a V read (4 bytes per lane, the two halves' rows 4 apart, 32
    // consecutive floats each) needs 4 * pitch = 32 (mod 64).
    constexpr int KP = D + 4;
    constexpr int VP = D + 8;
    __shared__ __attribute__((aligned(16))) float ks_lds[TK * KP];
    __shared__ __attribute__((aligned(16))) float vs_lds[TK * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int half = lane >> 5;

    const WorkItem wi = GROWS ? decode_grows_item(p, blockIdx.x, ROWS, TK)
                              : decode_band_item(p, xcd_contiguous(blockIdx.x, gridDim.x), TK);
    const KeyStream& ks = wi.ks;
    const int b = wi.b, kvh = wi.kvh;
    const int hq = kvh * p.group + wi.hg;  // one head per workgroup (hpw == 1)

    // ---- the lane's query row (column l32 of S^T) ------------------------------
    const int wave_row0 = wi.row0 + wave * 32;
    const int row = wave_row0 + l32;
    int qpos, qres;
    if (!GROWS) {
        qres = row;
        qpos = row < ks.Nr ? ks.r + row * ks.dil : -1;
    } else {
        qres = 0;
        qpos = row < p.n_global ? p.gpos[row] : -1;
    }
    SWA_DCHECK(qpos < p.N && hq < p.Hq && b < p.B);
    // a wave without rows (past the residue class, or past the global list)
    // still loads tiles and passes the barriers, but computes nothing
    const bool wave_idle = GROWS ? wave_row0 >= p.n_global : wave_row0 >= ks.Nr;
    f32x4 qreg[G];
    {
        const float* qp =
            (const float*)p.q + (((size_t)b * p.N + max(qpos, 0)) * p.Hq + hq) * D + half * 4;
#pragma unroll
        for (int g = 0; g < G; g++)
            qreg[g] = qpos >= 0 ? *(const f32x4*)(qp + 8 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] = f32x16{};
    float m_run = kEmptyMax, l_run = 0.f;   // l_run: the lane's half of the row sum
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
                SWA_DCHECK(kk >= -p.W && (unsigned)ring_slot(ks, kk, p.W) < (unsigned)p.W);
                const size_t o = (size_t)ring_slot(ks, kk, p.W) * D + c4 * 4;
                ksrc = krbase + o;
                vsrc = vrbase + o;
            } else {
                const int pos = key_position(ks, p, j, key, TK, GROWS);
                if (pos >= 0) {
                    SWA_DCHECK(pos < p.N);
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
            *(f32x4*)(ks_lds + key * KP + c4 * 4) = kv;
            *(f32x4*)(vs_lds + key * VP + c4 * 4) = vv;
        }
        __syncthreads();
        if (wave_idle) continue;

        // S^T = K Q^T: element e of the lane is key (e >> 2) * 8 + half * 4 + (e & 3)
        f32x16 s = f32x16{};
#pragma unroll
        for (int g = 0; g < G; g++) {
            const f32x4 kf = *(const f32x4*)(ks_lds + l32 * KP + 8 * g + 4 * half);
#pragma unroll
            for (int i = 0; i < 4; i++)
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[i], qreg[g][i], s, 0, 0, 0);
        }

        // element masks (every tile: this path serves small sizes)
        const bool band_tile = GROWS || j < ks.n_band_tiles;
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int k = (e >> 2) * 8 + half * 4 + (e & 3);
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
            s[e] = valid ? s[e] : -INFINITY;
            mx = fmaxf(mx, s[e]);
        }
        mx = wave_max_xor32(mx) * c;
        const bool up = mx > m_run + kLazyRescale;
        const float m_use = up ? mx : m_run;
        if (__any(up)) {
            const float alpha = fast_exp2(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; db++) oacc[db] *= alpha;
        }
        m_run = m_use;
        float pw[16];
#pragma unroll
        for (int e = 0; e < 16; e++) {
            pw[e] = fast_exp2(__builtin_fmaf(s[e], c, -m_use));
            l_run += pw[e];
        }

        // O^T += V^T P^T: step (g, jj) pairs keys 8g + jj (half 0) and 8g + 4 + jj (half 1)
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
            for (int g = 0; g < 4; g++)
#pragma unroll
                for (int jj = 0; jj < 4; jj++) {
                    const float va = vs_lds[(8 * g + 4 * half + jj) * VP + db * 32 + l32];
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, pw[4 * g + jj], oacc[db],
                                                                    0, 0, 0);
                }
    }

    // ---- epilogue: the lane holds dims db * 32 + (e >> 2) * 8 + half * 4 + (e & 3)
    const float l_tot = l_run + lane_xor32(l_run);
    if (wave_idle || qpos < 0) return;
    if (!GROWS) {
        const float inv = 1.0f / l_tot;
        float* op = (float*)p.out + (((size_t)b * p.N + qpos) * p.Hq + hq) * D + half * 4;
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                f32x4 o4;
#pragma unroll
                for (int i = 0; i < 4; i++) o4[i] = oacc[db][4 * g + i] * inv;
                *(f32x4*)(op + db * 32 + g * 8) = o4;
            }
        if (p.lse != nullptr && half == 0)
            p.lse[((size_t)b * p.Hq + hq) * p.N + qpos] =
                (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    } else {
        SWA_DCHECK(row < p.n_global && wi.chunk < p.g_nchunks);
        float* rec = p.partials +
                     ((((size_t)b * p.Hq + hq) * p.n_global + row) * p.g_nchunks + wi.chunk) *
                         (D + kPartialPad);
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                f32x4 o4;
#pragma unroll
                for (int i = 0; i < 4; i++) o4[i] = oacc[db][4 * g + i];
                *(f32x4*)(rec + db * 32 + g * 8 + half * 4) = o4;
            }
        if (half == 0) {
            rec[D] = m_run;
            rec[D + 1] = l_tot;
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

#ifdef SWA_DEBUG
SWA_DEBUG_COUNTER_READER(debug_counter_fwd_f32)
#endif

}  // namespace swa
