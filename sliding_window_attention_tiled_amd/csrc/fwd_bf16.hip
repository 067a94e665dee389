// fwd_bf16.hip -- sliding-window attention forward, bf16 inputs, gfx950 MFMA.
//
// Each workgroup (4 waves) owns a tile of query positions of one residue class
// r = i mod d for one kv head and `hpw` query heads of its group.  Inside a
// residue class the dilated window i + t*d (mhpn.cn "Dilated sliding window",
// section 2) is an ordinary window over m = (i - r) / d, so every gathered
// Q/K/V row is a whole contiguous head vector and the tiles stay dense
// (the block-level handling that page's section 4 asks for, at the finest
// granularity that keeps rows contiguous).
//
// The workgroup walks only the K/V tiles that intersect the union of its
// queries' windows (bmjup.com "Sliding window attention", section 3: cost
// O(n*W) instead of O(n^2)); element masks are applied only on tiles that
// straddle a window edge.  Scores are formed transposed, S^T = K * Q^T, on
// v_mfma_f32_32x32x16_bf16 so that each lane holds 32 keys of one query: the
// softmax row reductions are in-lane plus one exchange with lane ^ 32.  The
// probabilities are rounded to bf16 and multiplied with V^T, read from the
// natural-layout V tile through ds_read_b64_tr_b16.  The softmax is kept
// online (running max m, sum l, rescaled accumulator), with the max moved only
// when a tile exceeds it by more than 2^8, which is exact up to rounding.
//
// Global tokens (aiqz.cc "Sliding window attention: Mistral", section
// "global attention tokens"): after the band, a band workgroup also visits
// gathered tiles of the global keys, masking those already counted in the
// band (or in the future, for causal calls).  Global query rows are computed
// by the same kernel in GROWS mode: query rows are the gathered global
// positions, the keys are split into chunks and each chunk writes a partial
// (acc, m, l) that the combine kernel merges.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fwd_common.h"
#include "swa_kernels.h"

namespace swa {
namespace {

constexpr int BN = 64;        // keys per K/V tile
constexpr int NTHREADS = 256; // 4 waves

template <int D>
struct TileCfg {
    static constexpr int PITCH = D + 8;               // bf16 elements per LDS row
    static constexpr int ELEMS = BN * PITCH;          // one K or V tile
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int PER_THREAD = BN * CPR / NTHREADS;
    static_assert(PER_THREAD * NTHREADS == BN * CPR, "tile does not split evenly");
};

template <int D>
__device__ __forceinline__ void load_tile_regs(u32x4 (&kr)[TileCfg<D>::PER_THREAD],
                                               u32x4 (&vr)[TileCfg<D>::PER_THREAD],
                                               const __bf16* kbase, const __bf16* vbase,
                                               int rowstride, const KeyStream& ks,
                                               const FwdParams& p, int j, bool grows) {
    using T = TileCfg<D>;
#pragma unroll
    for (int u = 0; u < T::PER_THREAD; u++) {
        const int ci = threadIdx.x + u * NTHREADS;
        const int key = ci / T::CPR, c = ci % T::CPR;
        const int pos = key_position(ks, p, j, key, BN, grows);
        if (pos >= 0) {
            const size_t off = (size_t)pos * rowstride + c * 8;
            kr[u] = *(const u32x4*)(kbase + off);
            vr[u] = *(const u32x4*)(vbase + off);
        } else {
            kr[u] = u32x4{0u, 0u, 0u, 0u};
            vr[u] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile_lds(const u32x4 (&kr)[TileCfg<D>::PER_THREAD],
                                               const u32x4 (&vr)[TileCfg<D>::PER_THREAD],
                                               unsigned short* ks_lds, unsigned short* vs_lds) {
    using T = TileCfg<D>;
#pragma unroll
    for (int u = 0; u < T::PER_THREAD; u++) {
        const int ci = threadIdx.x + u * NTHREADS;
        const int key = ci / T::CPR, c = ci % T::CPR;
        *(u32x4*)(ks_lds + key * T::PITCH + c * 8) = kr[u];
        *(u32x4*)(vs_lds + key * T::PITCH + c * 8) = vr[u];
    }
}

// GROWS = false: band workgroups (plus global key columns).
// GROWS = true : global query rows over one key chunk, partial output.
template <int D, int QB, bool GROWS>
__global__ __launch_bounds__(NTHREADS, QB == 1 ? 2 : 1)
void swa_fwd_bf16_kernel(const FwdParams p) {
    using T = TileCfg<D>;
    constexpr int KC = D / 16;   // 16-deep k-steps of QK^T
    constexpr int DB = D / 32;   // 32-row blocks of O^T

    __shared__ __attribute__((aligned(16))) unsigned short smem[4 * T::ELEMS];
    // stage st: K tile at smem + 2*st*ELEMS, V tile right after it
    auto k_lds = [&](int st) { return smem + 2 * st * T::ELEMS; };
    auto v_lds = [&](int st) { return smem + (2 * st + 1) * T::ELEMS; };

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l32 = lane & 31;
    const int half = lane >> 5;

    // ---- work item ---------------------------------------------------------
    const WorkItem wi = GROWS ? decode_grows_item(p, blockIdx.x, (4 / p.hpw) * 32 * QB, BN)
                              : decode_band_item(p, xcd_contiguous(blockIdx.x, gridDim.x), BN);
    const int b = wi.b, kvh = wi.kvh, hg = wi.hg, chunk = wi.chunk;
    const KeyStream& ks = wi.ks;
    // wave_row0: residue coordinate (band) or global index (GROWS) of the wave's first row
    const int wave_row0 = wi.row0 + (wave / p.hpw) * 32 * QB;
    const int hq = kvh * p.group + hg * p.hpw + (wave % p.hpw);

    const int rowstride = p.Hkv * D;
    const __bf16* kbase = (const __bf16*)p.k + ((size_t)b * p.N * p.Hkv + kvh) * D;
    const __bf16* vbase = (const __bf16*)p.v + ((size_t)b * p.N * p.Hkv + kvh) * D;

    // ---- query rows of this wave (B operand of S^T = K Q^T) -------------------
    int qpos[QB];     // absolute position of the lane's query row, -1 if none
    int qres[QB];     // residue coordinate (band mode)
    bf16x8 qreg[QB][KC];
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
        const int row = wave_row0 + qb * 32 + l32;
        if (!GROWS) {
            qres[qb] = row;
            qpos[qb] = row < ks.Nr ? ks.r + row * ks.dil : -1;
        } else {
            qres[qb] = 0;
            qpos[qb] = row < p.n_global ? p.gpos[row] : -1;
        }
        const __bf16* qp = (const __bf16*)p.q +
                           (((size_t)b * p.N + max(qpos[qb], 0)) * p.Hq + hq) * D + half * 8;
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            if (qpos[qb] >= 0) {
                qreg[qb][kc] = *(const bf16x8*)(qp + kc * 16);
            } else {
                qreg[qb][kc] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
            }
        }
    }
    // wave row range in residue coordinates (band) for tile classification
    const int w_first = wave_row0;
    const int w_last_raw = wave_row0 + 32 * QB - 1;

    f32x16 oacc[QB][DB];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
        m_run[qb] = kEmptyMax;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; db++) oacc[qb][db] = f32x16{};
    }
    const float c = p.scale_log2;

    // ---- prologue: tile 0 into stage 0 ---------------------------------------
    u32x4 kr[T::PER_THREAD], vr[T::PER_THREAD];
    if (ks.n_tiles > 0) {
        load_tile_regs<D>(kr, vr, kbase, vbase, rowstride, ks, p, 0, GROWS);
        store_tile_lds<D>(kr, vr, k_lds(0), v_lds(0));
    }
    __syncthreads();

    for (int j = 0; j < ks.n_tiles; j++) {
        const int st = j & 1;
        const bool has_next = j + 1 < ks.n_tiles;
        if (has_next) load_tile_regs<D>(kr, vr, kbase, vbase, rowstride, ks, p, j + 1, GROWS);

        // classify this tile for this wave (wave-uniform)
        const bool band_tile = GROWS || j < ks.n_band_tiles;
        bool skip = false, need_mask = true;
        if (!GROWS && band_tile) {
            const int kt0 = ks.k_lo + j * BN;
            const int kt1 = kt0 + BN - 1;
            const int w_last = min(w_last_raw, ks.Nr - 1);
            skip = w_first > w_last || kt0 > w_last + p.wr || kt1 < w_first - p.wl;
            need_mask = !(kt0 >= w_last - p.wl && kt1 <= w_first + p.wr && kt1 <= ks.k_hi);
        }
        if (!skip) {
            const unsigned short* Ks = k_lds(st);
            const unsigned short* Vs = v_lds(st);
            // S^T = K Q^T : two 32-key blocks x QB 32-query blocks
            f32x16 s[QB][2];
#pragma unroll
            for (int qb = 0; qb < QB; qb++) {
                s[qb][0] = f32x16{};
                s[qb][1] = f32x16{};
            }
#pragma unroll
            for (int kc = 0; kc < KC; kc++) {
#pragma unroll
                for (int kb = 0; kb < 2; kb++) {
                    const bf16x8 a =
                        *(const bf16x8*)(Ks + (kb * 32 + l32) * T::PITCH + kc * 16 + half * 8);
#pragma unroll
                    for (int qb = 0; qb < QB; qb++)
                        s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][kc],
                                                                            s[qb][kb], 0, 0, 0);
                }
            }
            // element masks (edge tiles, global-key tiles, GROWS tiles)
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; kb++) {
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int koff = kb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
#pragma unroll
                        for (int qb = 0; qb < QB; qb++) {
                            bool valid;
                            if (GROWS) {
                                const int kk = ks.k_lo + j * BN + koff;
                                valid = kk <= ks.k_hi && qpos[qb] >= 0 &&
                                        (!p.causal || kk <= qpos[qb]);
                            } else if (band_tile) {
                                const int kk = ks.k_lo + j * BN + koff;
                                const int dl = kk - qres[qb];
                                valid = kk <= ks.k_hi && dl >= -p.wl && dl <= p.wr;
                            } else {
                                const int gi = (j - ks.n_band_tiles) * BN + koff;
                                valid = gi < ks.n_global && qpos[qb] >= 0 &&
                                        global_key_visible(p, ks, p.gpos[gi], qres[qb], qpos[qb]);
                            }
                            if (!valid) s[qb][kb][e] = -INFINITY;
                        }
                    }
                }
            }
            // online softmax
#pragma unroll
            for (int qb = 0; qb < QB; qb++) {
                float mx = s[qb][0][0];
#pragma unroll
                for (int e = 1; e < 16; e++) mx = fmaxf(mx, s[qb][0][e]);
#pragma unroll
                for (int e = 0; e < 16; e++) mx = fmaxf(mx, s[qb][1][e]);
                mx = wave_max_xor32(mx) * c;
                const bool up = mx > m_run[qb] + kLazyRescale;
                const float m_use = up ? mx : m_run[qb];
                if (__any(up)) {
                    const float alpha = fast_exp2(m_run[qb] - m_use);
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; db++) oacc[qb][db] *= alpha;
                }
                m_run[qb] = m_use;
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; kb++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const float pe = fast_exp2(__builtin_fmaf(s[qb][kb][e], c, -m_use));
                        s[qb][kb][e] = pe;
                        ls += pe;
                    }
                l_run[qb] += ls;
            }
            // O^T += V^T P^T : four 16-key steps
#pragma unroll
            for (int t = 0; t < 4; t++) {
                bf16x8 pb[QB];
#pragma unroll
                for (int qb = 0; qb < QB; qb++)
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        pb[qb][e] = (__bf16)s[qb][t >> 1][(t & 1) * 8 + e];
                const int key1 = t * 16 + half * 4 + ((lane & 15) >> 2);
                const int colo = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
                for (int db = 0; db < DB; db++) {
                    const int col = db * 32 + colo;
                    const i16x4 lo = lds_read_tr16(Vs + key1 * T::PITCH + col);
                    const i16x4 hi = lds_read_tr16(Vs + (key1 + 8) * T::PITCH + col);
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int qb = 0; qb < QB; qb++)
                        oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            a, pb[qb], oacc[qb][db], 0, 0, 0);
                }
            }
        }
        if (has_next) store_tile_lds<D>(kr, vr, k_lds(st ^ 1), v_lds(st ^ 1));
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------------
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
        if (qpos[qb] < 0) continue;
        if (!GROWS) {
            const float inv = 1.0f / l_tot;
            __bf16* op = (__bf16*)p.out + (((size_t)b * p.N + qpos[qb]) * p.Hq + hq) * D;
#pragma unroll
            for (int db = 0; db < DB; db++)
#pragma unroll
                for (int jq = 0; jq < 4; jq++) {
                    bf16x4 o4;
#pragma unroll
                    for (int e = 0; e < 4; e++) o4[e] = (__bf16)(oacc[qb][db][jq * 4 + e] * inv);
                    *(bf16x4*)(op + db * 32 + jq * 8 + half * 4) = o4;
                }
            if (p.lse != nullptr && half == 0)
                p.lse[((size_t)b * p.Hq + hq) * p.N + qpos[qb]] =
                    (m_run[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
        } else {
            const int gi = wave_row0 + qb * 32 + l32;
            float* rec = p.partials +
                         ((((size_t)b * p.Hq + hq) * p.n_global + gi) * p.g_nchunks + chunk) *
                             (D + kPartialPad);
#pragma unroll
            for (int db = 0; db < DB; db++)
#pragma unroll
                for (int jq = 0; jq < 4; jq++) {
                    f32x4 o4;
#pragma unroll
                    for (int e = 0; e < 4; e++) o4[e] = oacc[qb][db][jq * 4 + e];
                    *(f32x4*)(rec + db * 32 + jq * 8 + half * 4) = o4;
                }
            if (half == 0) {
                rec[D] = m_run[qb];
                rec[D + 1] = l_tot;
            }
        }
    }
}

template <int D, int QB>
hipError_t launch_d(const FwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL((swa_fwd_bf16_kernel<D, QB, false>), dim3(p.n_blocks), dim3(NTHREADS), 0,
                       s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_global == 0) return e;
    const int grid = p.B * p.Hkv * p.head_groups * p.g_rowgroups * p.g_nchunks;
    hipLaunchKernelGGL((swa_fwd_bf16_kernel<D, QB, true>), dim3(grid), dim3(NTHREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

int fwd_bf16_rows_per_wave() { return 32; }

hipError_t launch_fwd_bf16(const FwdParams& p, int D, hipStream_t s) {
    if (D == 128) return launch_d<128, 1>(p, s);
    return launch_d<64, 1>(p, s);
}

}  // namespace swa
