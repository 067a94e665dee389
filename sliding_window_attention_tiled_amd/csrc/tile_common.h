// tile_common.h -- K/V tile staging shared by the bf16 forward and backward
// kernels: the tile shape, its LDS pitches, and the load (global -> registers)
// and store (registers -> LDS) of one tile of a key stream.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fwd_common.h"
#include "swa_kernels.h"

namespace swa {

constexpr int BN = 64;        // keys per K/V tile
constexpr int kFarAway = -(1 << 30);  // residue coordinate outside every window

template <int D, int NW>
struct TileCfg {
    static constexpr int NT = 64 * NW;                          // threads per workgroup
    // LDS row pitches (bf16 elements).  K rows are read 16 B per lane, 16
    // rows per LDS cycle: a pitch of 4 (mod 64) dwords puts those rows on
    // distinct banks.  V rows are read by ds_read_b64_tr_b16, 4 consecutive
    // rows x 64 B per 32 lanes: a pitch of 16 or 48 (mod 64) dwords puts the
    // four rows on four distinct 16-bank quarters.  D + 32 elements is 48
    // dwords at D = 64 and 80 = 16 (mod 64) at D = 128.
    static constexpr int KP = D + 8;
    static constexpr int VP = D + 32;
    static constexpr int K_ELEMS = BN * KP;
    static constexpr int V_ELEMS = BN * VP;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int CPR = D / 8;                            // 16-byte chunks per row
    static constexpr int PER_THREAD = BN * CPR / NT;
    static constexpr int KEY_STEP = NT / CPR;                    // rows between a thread's chunks
    static_assert(PER_THREAD * NT == BN * CPR, "tile does not split evenly");
};

// Loads tile j of the key stream into registers (zero rows for padding).
// For gathered global-key tiles it also records, per key, the position and
// the residue coordinate g / d when g is in this residue class (else a value
// no window reaches) in gk[2][BN], for the element masks.  Band tiles that
// start at a negative coordinate (chunked prefill) take those keys from the
// ring rows krbase / vrbase (row pitch D).
// PLAIN: every tile is a run of rows of the key stream (no ring prefix, no
// gathered global keys), as in the global-row pass and in the band loop of a
// launch with global tokens (which has no ring).
template <class T, bool PLAIN>
__device__ __forceinline__ void load_tile(u32x4 (&kr)[T::PER_THREAD],
                                          u32x4 (&vr)[T::PER_THREAD],
                                          const __bf16* kbase, const __bf16* vbase,
                                          const __bf16* krbase, const __bf16* vrbase,
                                          int rowstride, const KeyStream& ks, const FwdParams& p,
                                          int j, int* gk, const int* gpos) {
    const int key0 = threadIdx.x / T::CPR;
    const int c = threadIdx.x % T::CPR;
    if (!PLAIN && j < ks.n_band_tiles && ks.k_lo + j * BN < 0) {
        // d = 1 and r = 0 here: coordinate = position within the chunk
        const int kk0 = ks.k_lo + j * BN + key0;
#pragma unroll
        for (int u = 0; u < T::PER_THREAD; u++) {
            const int kk = kk0 + u * T::KEY_STEP;
            const __bf16* ks_src = nullptr;
            const __bf16* vs_src = nullptr;
            if (kk < 0) {
                SWA_DCHECK(kk >= -p.W && (unsigned)ring_slot(ks, kk, p.W) < (unsigned)p.W);
                const size_t off = (size_t)ring_slot(ks, kk, p.W) * T::CPR * 8 + c * 8;
                ks_src = krbase + off;
                vs_src = vrbase + off;
            } else if (kk <= ks.k_hi) {
                SWA_DCHECK(kk < p.N);
                const size_t off = (size_t)kk * rowstride + c * 8;
                ks_src = kbase + off;
                vs_src = vbase + off;
            }
            kr[u] = ks_src ? *(const u32x4*)ks_src : u32x4{0u, 0u, 0u, 0u};
            vr[u] = vs_src ? *(const u32x4*)vs_src : u32x4{0u, 0u, 0u, 0u};
        }
        return;
    }
    if (PLAIN || j < ks.n_band_tiles) {
        // band keys past k_hi only occur in the last tile, which is always
        // element-masked: load them from k_hi instead of predicating the loads
        const int kk0 = ks.k_lo + j * BN + key0;
#pragma unroll
        for (int u = 0; u < T::PER_THREAD; u++) {
            const int kk = min(kk0 + u * T::KEY_STEP, ks.k_hi);
            SWA_DCHECK(kk >= 0 && ks.r + kk * ks.dil < p.N);
            const size_t off = (size_t)(ks.r + kk * ks.dil) * rowstride + c * 8;
            kr[u] = *(const u32x4*)(kbase + off);
            vr[u] = *(const u32x4*)(vbase + off);
        }
        return;
    }
    int kpos[T::PER_THREAD];
    {
        const int g0 = (j - ks.n_band_tiles) * BN + key0;
#pragma unroll
        for (int u = 0; u < T::PER_THREAD; u++) {
            const int gi = g0 + u * T::KEY_STEP;
            kpos[u] = gi < ks.n_global ? gpos[gi] : -1;
            if (c == 0) {
                const int g = kpos[u];
                gk[key0 + u * T::KEY_STEP] = g;
                gk[BN + key0 + u * T::KEY_STEP] =
                    (g >= 0 && g % ks.dil == ks.r) ? g / ks.dil : kFarAway;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < T::PER_THREAD; u++) {
        if (kpos[u] >= 0) {
            SWA_DCHECK(kpos[u] < p.N);
            const size_t off = (size_t)kpos[u] * rowstride + c * 8;
            kr[u] = *(const u32x4*)(kbase + off);
            vr[u] = *(const u32x4*)(vbase + off);
        } else {
            kr[u] = u32x4{0u, 0u, 0u, 0u};
            vr[u] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

template <class T>
__device__ __forceinline__ void store_tile(const u32x4 (&kr)[T::PER_THREAD],
                                           const u32x4 (&vr)[T::PER_THREAD],
                                           unsigned short* stage) {
    const int key0 = threadIdx.x / T::CPR;
    const int c = threadIdx.x % T::CPR;
#pragma unroll
    for (int u = 0; u < T::PER_THREAD; u++) {
        const int key = key0 + u * T::KEY_STEP;
        SWA_DCHECK(key < BN);
        *(u32x4*)(stage + key * T::KP + c * 8) = kr[u];
        *(u32x4*)(stage + T::K_ELEMS + key * T::VP + c * 8) = vr[u];
    }
}

}  // namespace swa
