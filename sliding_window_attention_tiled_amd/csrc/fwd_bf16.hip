// fwd_bf16.hip -- sliding-window attention forward, bf16 inputs, gfx950 MFMA.
//
// Each workgroup owns a tile of query positions of one residue class r = i mod
// d for one kv head and `hpw` query heads of its group: eight waves when four
// query heads share the kv head (two 32-position row blocks per head, so every
// K/V tile staged in LDS serves 256 query rows), four waves otherwise.  Each
// wave holds 32 query rows of one head.  Inside a
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
// natural-layout V tile through ds_read_b64_tr_b16.  K fragments are read
// from LDS in batches ahead of their MFMAs, and a step's V fragments ahead of
// its exponentials, so LDS latency overlaps other work.  The softmax is kept
// online (running max m, sum l, rescaled accumulator), with the max moved only
// when a tile exceeds it by more than 2^8, which is exact up to rounding; the
// running sum adds the bf16-rounded weights, the same ones the products with
// V use, so out is normalised by exactly the weights it was built from.
//
// Global tokens (aiqz.cc "Sliding window attention: Mistral", section
// "global attention tokens"): after the band, a band workgroup also visits
// gathered tiles of the global keys, masking those already counted in the
// band (or in the future, for causal calls).  Global query rows are computed
// by the same kernel in GROWS mode: query rows are the gathered global
// positions, the keys are split into chunks and each chunk writes a partial
// (acc, m, l) that the combine kernel merges.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "fwd_common.h"
#include "swa_kernels.h"
#include "tile_common.h"


namespace swa {
namespace {

constexpr int kQB = 1;  // 32-query blocks per wave

// GROWS = false: band workgroups, with gathered tiles of the global keys
//                after the band when GLOB.
// GROWS = true : global query rows over one key chunk, partial output.
// Waves per SIMD the register allocation must leave room for.  Four-wave
// workgroups with one 32-row block per wave: two at D = 128 (two workgroups
// per CU), three at D = 64, where three workgroups' tiles fit in LDS and the
// kernel fits in 168 registers without spilling.
template <int D, int QB, int NW>
constexpr int kFwdWavesPerSimd = (QB == 1 && NW == 4) ? (D == 64 ? 3 : 2) : 1;

template <int D, int QB, int NW, bool GROWS, bool GLOB>
__global__ __launch_bounds__(64 * NW, (kFwdWavesPerSimd<D, QB, NW>))
void swa_fwd_bf16_kernel(const FwdParams p) {
    constexpr bool kGathered = GLOB && !GROWS;
    using T = TileCfg<D, NW>;
    constexpr int KC = D / 16;   // 16-deep k-steps of QK^T
    constexpr int DB = D / 32;   // 32-row blocks of O^T

    __shared__ __attribute__((aligned(16))) unsigned short smem[2 * T::STAGE];
    __shared__ __attribute__((aligned(16))) int gk_lds[2][2 * BN];
    // the global positions, read by the gathered-key tile loads.  Kept in LDS:
    // a per-lane load from the parameter block inside the tile loop would be a
    // vector-memory write that the compiler waits for before the next LDS read.
    __shared__ int gpos_lds[SWA_MAX_GLOBAL];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l32 = lane & 31;
    const int half = lane >> 5;

    // ---- work item ---------------------------------------------------------
    const WorkItem wi = GROWS ? decode_grows_item(p, blockIdx.x, (NW / p.hpw) * 32 * QB, BN)
                              : decode_band_item(p, xcd_contiguous(blockIdx.x, gridDim.x), BN);
    const int b = wi.b, kvh = wi.kvh, hg = wi.hg, chunk = wi.chunk;
    const KeyStream& ks = wi.ks;
    // residue coordinate (band) or global index (GROWS) of the wave's first row
    const int wave_row0 = wi.row0 + (wave / p.hpw) * 32 * QB;
    const int hq = kvh * p.group + hg * p.hpw + (wave % p.hpw);

    const int rowstride = p.Hkv * D;
    const __bf16* kbase = (const __bf16*)p.k + ((size_t)b * p.N * p.Hkv + kvh) * D;
    const __bf16* vbase = (const __bf16*)p.v + ((size_t)b * p.N * p.Hkv + kvh) * D;
    // ring rows of this (b, kv head) for chunked prefill (unused otherwise)
    const size_t ring_off = ((size_t)b * p.Hkv + kvh) * (size_t)p.W * D;
    const __bf16* krbase = (const __bf16*)p.kring + ring_off;
    const __bf16* vrbase = (const __bf16*)p.vring + ring_off;

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
        SWA_DCHECK(qpos[qb] < p.N && hq < p.Hq && b < p.B);
        const __bf16* qp = (const __bf16*)p.q +
                           (((size_t)b * p.N + max(qpos[qb], 0)) * p.Hq + hq) * D + half * 8;
#pragma unroll
        for (int kc = 0; kc < KC; kc++)
            qreg[qb][kc] = qpos[qb] >= 0 ? *(const bf16x8*)(qp + kc * 16)
                                         : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    const int w_first = wave_row0;
    const int w_last = min(wave_row0 + 32 * QB - 1, ks.Nr - 1);

    f32x16 oacc[QB][DB];
    float m_run[QB], l_run[QB];   // l_run: the lane's half of the row sum (dot2)
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
        m_run[qb] = kEmptyMax;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; db++) oacc[qb][db] = f32x16{};
    }
    const float c = p.scale_log2;
    const __bf16 one = (__bf16)1.0f;
    const bf16x2 ones = {one, one};

    // ---- prologue: tile 0 into stage 0 ---------------------------------------
    // (tile 0 is a band tile: the barrier below publishes gpos_lds before the
    // first gathered-key tile is loaded)
    if (kGathered)
        for (int i = threadIdx.x; i < p.n_global; i += T::NT) gpos_lds[i] = p.gpos[i];
    // With p.rotate the band tiles are walked in a rotated order: step j
    // takes the band tile whose absolute index (k_lo / BN + tile) is j modulo
    // the band's tile count.  Workgroups whose bands have the same length then
    // read the same K/V tile at the same step, while it is in L2, instead of a
    // few steps apart.  Gathered global-key tiles follow in order.
    // (compiled only into the launches the host may rotate: four-wave
    // workgroups at D = 128; the others keep the plain order at no cost)
    constexpr bool kRotatable = !GROWS && D == 128 && NW == 4;
    const int nbt = ks.n_band_tiles;
    int rot = 0;
    if (kRotatable && nbt > 0 && p.rotate) {
        const int a = ks.k_lo >= 0 ? ks.k_lo / BN : -((-ks.k_lo + BN - 1) / BN);
        rot = ((-a) % nbt + nbt) % nbt;
    }
    auto tile_at = [&](int j) {
        if constexpr (!kRotatable) return j;
        const int t = j + rot;   // < 2 * nbt for a band step
        return j < nbt ? (t >= nbt ? t - nbt : t) : j;
    };
    u32x4 kr[T::PER_THREAD], vr[T::PER_THREAD];
    if (ks.n_tiles > 0) {
        load_tile<T, GROWS>(kr, vr, kbase, vbase, krbase, vrbase, rowstride, ks, p, tile_at(0),
                            gk_lds[0], gpos_lds);
        store_tile<T>(kr, vr, smem);
    }
    __syncthreads();


    // One step of the key stream: tile j in stage j & 1.  GATH: tile j is a
    // gathered global-key tile (compile time), so that the band tiles run a
    // loop with only the band masks and band loads, and the gathered tiles
    // (after the band) a copy with only theirs: one loop body for both kept
    // every path's values live across the band and took more registers than
    // the band needs.  The band loop does not prefetch the first gathered
    // tile; its step loads it.  (Launches with global tokens have no ring
    // prefix, so the band loads there are plain row loads.)
    const int n_main = kGathered ? min(ks.n_band_tiles, ks.n_tiles) : ks.n_tiles;
    auto step = [&](const int j, auto gath_tag) {
        constexpr bool GATH = decltype(gath_tag)::value;
        constexpr bool kBandLoads = GROWS || (kGathered && !GATH);
        const int st = j & 1;
        const bool has_next = j + 1 < (GATH ? ks.n_tiles : n_main);
        if constexpr (GATH) {
            if (j == n_main) {
                load_tile<T, GROWS>(kr, vr, kbase, vbase, krbase, vrbase, rowstride, ks, p,
                                    tile_at(j), gk_lds[st], gpos_lds);
                store_tile<T>(kr, vr, smem + st * T::STAGE);
                __syncthreads();
            }
        }

        // classify this tile for this wave (wave-uniform)
        const int jt = tile_at(j);
        constexpr bool band_tile = !GATH;
        const int kt0 = ks.k_lo + jt * BN;
        bool skip = false, need_mask = true;
        // a gathered tile with at most 32 entries: its second 32-key block is
        // padding, skipped
        const int gi0 = (jt - ks.n_band_tiles) * BN;   // list index of a gathered tile's key 0
        const bool half_tile = kGathered && !band_tile && p.n_global - gi0 <= 32;
        if (!GROWS && band_tile) {
            const int kt1 = kt0 + BN - 1;
            skip = w_first > w_last || kt0 > w_last + p.wr || kt1 < w_first - p.wl;
            need_mask = !(kt0 >= w_last - p.wl && kt1 <= w_first + p.wr && kt1 <= ks.k_hi);
        }
        // global-row mode: a wave past the last global row has nothing to compute
        // (with few global tokens most waves of the workgroup)
        if (GROWS) skip = wave_row0 >= p.n_global;
        const unsigned short* Ks = smem + st * T::STAGE;
        const unsigned short* Vs = Ks + T::K_ELEMS;
        f32x16 s[QB][2];
        float m_use[QB];
        if (!skip) {
            // S^T = K Q^T : two 32-key blocks x QB 32-query blocks
#pragma unroll
            for (int qb = 0; qb < QB; qb++) {
                s[qb][0] = f32x16{};
                s[qb][1] = f32x16{};
            }
            // K fragments are read in batches of KBATCH ahead of their MFMAs so
            // that LDS latency overlaps the matrix work (batches of 8 at D = 128
            // were 2.5% faster than 16: fewer registers held by fragments)
            constexpr int KBATCH = 2 * KC < 8 ? 2 * KC : 8;
            if (half_tile) {
#pragma unroll
                for (int qb = 0; qb < QB; qb++)
#pragma unroll
                    for (int e = 0; e < 16; e++) s[qb][1][e] = -INFINITY;
#pragma unroll
                for (int kc = 0; kc < KC; kc++) {
                    const bf16x8 a = *(const bf16x8*)(Ks + l32 * T::KP + kc * 16 + half * 8);
#pragma unroll
                    for (int qb = 0; qb < QB; qb++)
                        s[qb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][kc],
                                                                           s[qb][0], 0, 0, 0);
                }
            } else
#pragma unroll
            for (int k0 = 0; k0 < KC; k0 += KBATCH / 2) {
                bf16x8 a[KBATCH];
#pragma unroll
                for (int i = 0; i < KBATCH; i++) {
                    const int kc = k0 + i / 2, kb = i % 2;
                    a[i] = *(const bf16x8*)(Ks + (kb * 32 + l32) * T::KP + kc * 16 + half * 8);
                }
#pragma unroll
                for (int i = 0; i < KBATCH; i++) {
                    const int kc = k0 + i / 2, kb = i % 2;
#pragma unroll
                    for (int qb = 0; qb < QB; qb++)
                        s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qreg[qb][kc],
                                                                            s[qb][kb], 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, KBATCH, 0);       // DS reads first
                __builtin_amdgcn_sched_group_barrier(0x008, KBATCH * QB, 0);  // then MFMAs
            }
        }
        // Next tile into registers, issued after the score MFMAs: a load issued
        // before them makes the compiler wait for it ahead of the first MFMA
        // (their results may reuse the loads' address registers).  The loads
        // then overlap the softmax and P V, and are stored after them.
        SWA_DEBUG_BARRIER();   // every wave's score reads of this stage are done
        if (has_next)
            load_tile<T, kBandLoads>(kr, vr, kbase, vbase, krbase, vrbase, rowstride, ks, p,
                                     tile_at(j + 1), gk_lds[st ^ 1], gpos_lds);
        if (!skip) {
            // Element masks.  Lane key offsets within the tile are
            // kb*32 + (e>>2)*8 + half*4 + (e&3); all compares are per element.
            if (need_mask) {
                if (GROWS) {
#pragma unroll
                    for (int qb = 0; qb < QB; qb++) {
                        const int hi = p.causal ? min(ks.k_hi, qpos[qb]) : ks.k_hi;
                        const int lim = hi - kt0 - half * 4;  // valid when offset <= lim
#pragma unroll
                        for (int kb = 0; kb < 2; kb++)
#pragma unroll
                            for (int e = 0; e < 16; e++) {
                                const int ko = kb * 32 + (e >> 2) * 8 + (e & 3);
                                const int bad = (lim - ko) >> 31;
                                s[qb][kb][e] += __builtin_bit_cast(float, bad & 0xff800000);
                            }
                    }
                } else if (band_tile) {
#pragma unroll
                    for (int qb = 0; qb < QB; qb++) {
                        // x = key - query + wl must lie in [0, wl + wr] and the key
                        // must not pass k_hi: for this lane the valid offsets ko
                        // (less the lane's half * 4) form one interval [lo, hi], an
                        // empty one moved past the tile.  Per element one
                        // unsigned range compare and a select.
                        const int base = kt0 + half * 4 - qres[qb] + p.wl;
                        int lo = -base;
                        int hi = min(p.wl + p.wr - base, ks.k_hi - kt0 - half * 4);
                        if (hi < lo) lo = hi = 1 << 20;
                        const unsigned span = (unsigned)(hi - lo);
#pragma unroll
                        for (int kb = 0; kb < 2; kb++)
#pragma unroll
                            for (int e = 0; e < 16; e++) {
                                const int ko = kb * 32 + (e >> 2) * 8 + (e & 3);
                                if ((unsigned)(ko - lo) > span) s[qb][kb][e] = -INFINITY;
                            }
                    }
                } else {
                    // gathered global keys: visible unless already in the band,
                    // and (causal) not after the query
                    const int* gk = gk_lds[st];
                    const int span = p.wl + p.wr;
                    const int causal_mask = p.causal ? -1 : 0;
#pragma unroll
                    for (int kb = 0; kb < 2; kb++)
#pragma unroll
                        for (int e4 = 0; e4 < 4; e4++) {
                            const int4 g4 = *(const int4*)(gk + kb * 32 + e4 * 8 + half * 4);
                            const int4 r4 = *(const int4*)(gk + BN + kb * 32 + e4 * 8 + half * 4);
                            const int gv[4] = {g4.x, g4.y, g4.z, g4.w};
                            const int rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                            for (int e3 = 0; e3 < 4; e3++) {
#pragma unroll
                                for (int qb = 0; qb < QB; qb++) {
                                    // hidden when padding (g < 0), already in the band
                                    // (0 <= x <= span), or causal and after the query;
                                    // integer arithmetic only, as for the band masks
                                    const int x = rv[e3] - qres[qb] + p.wl;
                                    const int inband = ~(x | (span - x)) >> 31;
                                    const int future = causal_mask & ((qpos[qb] - gv[e3]) >> 31);
                                    const int bad = (gv[e3] >> 31) | inband | future;
                                    s[qb][kb][e4 * 4 + e3] +=
                                        __builtin_bit_cast(float, bad & 0xff800000);
                                }
                            }
                        }
                }
            }
            // online softmax: running max first, then per 16-key step the bf16
            // weights (B operand of P V) and their sum
#pragma unroll
            for (int qb = 0; qb < QB; qb++) {
                // the lane's own 32 keys first: only if some lane of the wave
                // passes the running max by more than the lazy bound is the max
                // exchanged with lane ^ 32 (otherwise every row keeps its max,
                // as the exchanged max would have decided too)
                float lmx = s[qb][0][0];
#pragma unroll
                for (int e = 1; e < 16; e++) lmx = fmaxf(lmx, s[qb][0][e]);
#pragma unroll
                for (int e = 0; e < 16; e++) lmx = fmaxf(lmx, s[qb][1][e]);
                if (__any(lmx * c > m_run[qb] + kLazyRescale)) {
                    const float mx = wave_max_xor32(lmx) * c;
                    const float m_new = mx > m_run[qb] + kLazyRescale ? mx : m_run[qb];
                    const float alpha = fast_exp2(m_run[qb] - m_new);
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; db++) oacc[qb][db] *= alpha;
                    m_run[qb] = m_new;
                }
                m_use[qb] = m_run[qb];
            }
            // O^T += V^T P^T : four 16-key steps; V^T through transposing reads
            // At D = 128 a wave takes issue priority over the other wave on its
            // SIMD while it runs P V, so that the other wave's softmax work
            // fills the gaps between these MFMAs rather than the reverse
            // (2% faster there; 2% slower at D = 64, where P V is short).
            if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
            const int key_l = half * 4 + ((lane & 15) >> 2);
            const int col_l = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                if (t >= 2 && half_tile) break;   // keys 32..63: padding, weight 0
                // V^T fragments of this step first: their LDS latency overlaps the
                // exponentials below
                bf16x8 va[DB];
#pragma unroll
                for (int db = 0; db < DB; db++) {
                    const unsigned short* vp = Vs + (t * 16 + key_l) * T::VP + db * 32 + col_l;
                    const i16x4 lo = lds_read_tr16(vp);
                    const i16x4 hi = lds_read_tr16(vp + 8 * T::VP);
                    va[db] = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
                bf16x8 pb[QB];
#pragma unroll
                for (int qb = 0; qb < QB; qb++) {
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        pb[qb][e] = (__bf16)fast_exp2(
                            __builtin_fmaf(s[qb][t >> 1][(t & 1) * 8 + e], c, -m_use[qb]));
                    float ls = l_run[qb];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const bf16x2 pr = {pb[qb][2 * e], pb[qb][2 * e + 1]};
                        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls, false);
                    }
                    l_run[qb] = ls;
                }
#pragma unroll
                for (int db = 0; db < DB; db++)
#pragma unroll
                    for (int qb = 0; qb < QB; qb++)
                        oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            va[db], pb[qb], oacc[qb][db], 0, 0, 0);
            }
        }
        if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
        SWA_DEBUG_BARRIER();   // every wave's P V reads of this stage are done
        if (has_next) store_tile<T>(kr, vr, smem + (st ^ 1) * T::STAGE);
        __syncthreads();
    };
    for (int j = 0; j < n_main; j++) step(j, std::false_type{});
    if constexpr (kGathered)
        for (int j = n_main; j < ks.n_tiles; j++) step(j, std::true_type{});

    // ---- epilogue ---------------------------------------------------------------
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
        const float l_tot = l_run[qb] + lane_xor32(l_run[qb]);
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
            SWA_DCHECK(gi < p.n_global && chunk < p.g_nchunks);
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

template <int D, int QB, int NW>
hipError_t launch_d(const FwdParams& p, hipStream_t s) {
    if (p.n_global == 0) {
        hipLaunchKernelGGL((swa_fwd_bf16_kernel<D, QB, NW, false, false>), dim3(p.n_blocks),
                           dim3(64 * NW), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((swa_fwd_bf16_kernel<D, QB, NW, false, true>), dim3(p.n_blocks),
                       dim3(64 * NW), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int grid = p.B * p.Hkv * p.head_groups * p.g_rowgroups * p.g_nchunks;
    hipLaunchKernelGGL((swa_fwd_bf16_kernel<D, QB, NW, true, false>), dim3(grid), dim3(64 * NW),
                       0, s, p);
    return hipGetLastError();
}

// Waves per workgroup: eight when four query heads share the K/V tiles (the
// tiles then serve two 32-position row blocks of each head), else four.
int waves_per_wg(int hpw) { return hpw == 4 ? 8 : 4; }

}  // namespace

FwdShape fwd_bf16_shape(int group) {
    // heads of one GQA group share the K/V tiles of a workgroup
    const int hpw = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
    const int rows = (waves_per_wg(hpw) / hpw) * 32 * kQB;
    return FwdShape{hpw, rows, rows};
}

hipError_t launch_fwd_bf16(const FwdParams& band, int D, hipStream_t s) {
    FwdParams p = band;
    const bool w8 = waves_per_wg(p.hpw) == 8;
    // In the natural order a workgroup reads a key tile bmq / BN steps after
    // its neighbour did, and in between the workgroups running on one XCD (32
    // CUs, one eight-wave or two four-wave workgroups each) read that many
    // steps' tiles.  Where that reaches the XCD's 4 MB L2 the tile is fetched
    // again, and the walk is rotated: four-wave workgroups of 128 positions at
    // D = 128 (2 steps x 64 workgroups x 32 KB).  Below it the natural order
    // already finds its tiles in L2 and is kept.
    constexpr double kL2Bytes = 4.0 * 1024 * 1024;
    const double reuse = (double)(p.bmq / BN) * (32 * (w8 ? 1 : 2)) * ((double)BN * D * 2 * 2);
    p.rotate = reuse >= kL2Bytes;
    if (fwd_pp_applies(p, D)) return launch_fwd_pp(p, s);
    if (D == 128) return w8 ? launch_d<128, kQB, 8>(p, s) : launch_d<128, kQB, 4>(p, s);
    return w8 ? launch_d<64, kQB, 8>(p, s) : launch_d<64, kQB, 4>(p, s);
}

#ifdef SWA_DEBUG
SWA_DEBUG_COUNTER_READER(debug_counter_fwd_bf16)
#endif

}  // namespace swa
