// bwd_bf16.hip -- backward of the sliding-window attention forward, bf16
// inputs, gfx950 MFMA.
//
// The gradients follow from the chain rule through s = scale q.k, the softmax
// over the attended set and the weighted sum of v (training with windowed
// attention: bmjup.com "Sliding window attention", Q&A on training vs
// inference; intelliparadigm.com section 5.1).  With P_ij = exp2(s_ij c -
// lse2_i) rebuilt from the forward's log-sum-exp, dP_ij = dout_i . v_j and
// delta_i = dout_i . out_i (= sum_j P_ij dP_ij):
//   dS_ij = P_ij (dP_ij - delta_i)
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i
// Three launches, no atomics:
//   1. delta per query row;
//   2. query-major (the forward's work items and key tiles): S^T = K Q^T,
//      dP^T = V dout^T, then dq^T += K^T dS^T, with K^T read transposed from
//      the K tile;
//   3. key-major: a workgroup owns 128 keys of one kv head and walks the query
//      positions whose windows reach them, for every query head of the group:
//      S = Q K^T and dP = dout V^T with keys on the lanes, then
//      dv^T += dout^T P and dk^T += Q^T dS, with dout^T and Q^T read
//      transposed from LDS.
// Both passes rebuild P from lse instead of a running softmax, so a key tile
// needs no rescaling.  P and dS enter the MFMAs rounded to bf16.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "fwd_common.h"
#include "swa_kernels.h"
#include "tile_common.h"

namespace swa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Transposed operands (K^T in the dq pass, dout^T and Q^T in the dk/dv pass)
// are read with ds_read_b64_tr_b16 from tiles whose row pitch is 4 (mod 64)
// dwords, the pitch that keeps the 16-byte row reads of the same tiles free of
// bank conflicts.  In one such read, 32 lanes fetch 4 rows x 8 chunks of 8
// bytes.  Taking the rows {0, 1, 8, 9} of a 16-row step (the high read: 2 rows
// further) and chunks at dword offsets {0, 2, 8, 10, 16, 18, 24, 26} places
// the 32 chunks on 64 distinct banks.  The B operand's k slots follow the same
// row order (slot_elem), and the accumulator rows follow the chunks (acc_dim).
__device__ __forceinline__ int tr_row(int lane) {
    const int e4 = (lane & 15) >> 2;
    return (lane >> 5) * 4 + (e4 & 1) + (e4 >> 1) * 8;
}
__device__ __forceinline__ int tr_col(int lane) {
    const int c = lane & 3;
    return 32 * ((lane >> 4) & 1) + 16 * (c >> 1) + 4 * (c & 1);
}
constexpr int tr_block_col(int db) { return 8 * (db & 1) + 64 * (db >> 1); }
constexpr int kTrHi = 2;
// element (0..7 of a 16-row step of an MFMA result block) that fills B slot e
constexpr int slot_elem(int e) { return (e & 1) | ((e & 2) << 1) | ((e & 4) >> 1); }
// head dimension of accumulator element 4 * jq + e of block db on lane half h
__device__ __forceinline__ int acc_dim(int db, int jq, int h) {
    return tr_block_col(db) + 16 * jq + 4 * h;
}

// ---- 1. delta_i = dout_i . out_i ---------------------------------------------------
// The float32 path's pass (the bf16 dq pass computes delta for its rows).
// D/8 lanes per row (8 elements each), 256 threads.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* out, const T* dout, float* delta,
                                                        int Hq, int N, int64_t rows) {
    constexpr int LPR = D / 8;
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const T* o = out + row * D + part * 8;
        const T* g = dout + row * D + part * 8;
#pragma unroll
        for (int e = 0; e < 8; e++) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
    if (row < rows && part == 0) {
        // row = (b * N + i) * Hq + h  ->  delta[(b * Hq + h) * N + i]
        const int h = (int)(row % Hq);
        const int64_t bi = row / Hq;
        const int64_t b = bi / N, i = bi % N;
        delta[(b * Hq + h) * N + i] = acc;
    }
}

// ---- 2. dq: query-major ----------------------------------------------------------
// The dq pass reads V by rows only (dP^T = V dout^T), so its V tile takes the K
// tile's pitch.
template <int D, int NW>
struct DqTileCfg : TileCfg<D, NW> {
    static constexpr int VP = TileCfg<D, NW>::KP;
    static constexpr int V_ELEMS = BN * VP;
    static constexpr int STAGE = TileCfg<D, NW>::K_ELEMS + V_ELEMS;
};

// Two workgroups per CU: the cap of 256 registers per lane costs a few spills,
// which the second resident workgroup more than hides.
// GLOB: after the band, gathered tiles of the global keys add the pairs of a
// row that is not itself global with the global keys outside its band (and,
// causal, not after it).  A global row's pairs outside its band are the
// global-row pass's.
template <int D, int NW, bool GLOB>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_bf16_kernel(const BwdParams bp) {
    using T = DqTileCfg<D, NW>;
    const FwdParams& p = bp.f;
    constexpr int KC = D / 16;   // 16-deep k-steps of the D contractions
    constexpr int DB = D / 32;   // 32-row blocks of dq^T

    __shared__ __attribute__((aligned(16))) unsigned short smem[2 * T::STAGE];
    __shared__ __attribute__((aligned(16))) int gk_lds[2][2 * BN];
    // the global positions for the gathered tile loads (an LDS copy: read
    // per lane from the parameter block inside the loop, they would add a
    // wait for vector memory before the next LDS read)
    __shared__ int gpos_lds[GLOB ? SWA_MAX_GLOBAL : 1];
    const int* gpos_ptr = GLOB ? gpos_lds : nullptr;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l32 = lane & 31;
    const int half = lane >> 5;

    const WorkItem wi = decode_band_item(p, xcd_contiguous(blockIdx.x, gridDim.x), BN);
    const int b = wi.b, kvh = wi.kvh, hg = wi.hg;
    const KeyStream& ks = wi.ks;
    const int wave_row0 = wi.row0 + (wave / p.hpw) * 32;
    const int hq = kvh * p.group + hg * p.hpw + (wave % p.hpw);

    const int rowstride = p.Hkv * D;
    const __bf16* kbase = (const __bf16*)p.k + ((size_t)b * p.N * p.Hkv + kvh) * D;
    const __bf16* vbase = (const __bf16*)p.v + ((size_t)b * p.N * p.Hkv + kvh) * D;

    // the lane's query row: q and dout as B operands, lse and delta
    const int row = wave_row0 + l32;
    const int qres = row;
    const int qpos = row < ks.Nr ? ks.r + row * ks.dil : -1;
    bf16x8 qreg[KC], greg[KC];
    {
        const size_t qo = (((size_t)b * p.N + max(qpos, 0)) * p.Hq + hq) * D + half * 8;
        const __bf16* qp = (const __bf16*)p.q + qo;
        const __bf16* gp = (const __bf16*)bp.dout + qo;
        const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            qreg[kc] = qpos >= 0 ? *(const bf16x8*)(qp + kc * 16) : z;
            greg[kc] = qpos >= 0 ? *(const bf16x8*)(gp + kc * 16) : z;
        }
    }
    const size_t lrow = ((size_t)b * p.Hq + hq) * p.N + max(qpos, 0);
    const float lse2 = qpos >= 0 ? p.lse[lrow] * kLog2e : 0.f;
    // delta = dout . out of the lane's row, from its half of the row (the
    // dout fragments above) and the other half's lane; every query row has
    // one owner lane pair in this pass, which writes it for the dk/dv pass
    // and the global-token passes that run after it
    float dlt;
    {
        const __bf16* op = (const __bf16*)bp.out +
                           (((size_t)b * p.N + max(qpos, 0)) * p.Hq + hq) * D + half * 8;
        float acc = 0.f;
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            const bf16x8 o = qpos >= 0 ? *(const bf16x8*)(op + kc * 16)
                                       : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
            for (int e = 0; e < 8; e++) acc = __builtin_fmaf((float)o[e], (float)greg[kc][e], acc);
        }
        dlt = acc + lane_xor32(acc);
        if (qpos >= 0 && half == 0) bp.delta[lrow] = dlt;
    }
    const int w_first = wave_row0;
    const int w_last = min(wave_row0 + 31, ks.Nr - 1);

    f32x16 dqacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) dqacc[db] = f32x16{};
    const float c = p.scale_log2;

    u32x4 kr[T::PER_THREAD], vr[T::PER_THREAD];
    if constexpr (GLOB)
        for (int i = threadIdx.x; i < p.n_global; i += T::NT) gpos_lds[i] = p.gpos[i];
    // (tile 0 is a band tile: the gathered loads that read gpos_lds come after
    // the barrier below)
    if (ks.n_tiles > 0) {
        load_tile<T, false>(kr, vr, kbase, vbase, kbase, vbase, rowstride, ks, p, 0, gk_lds[0],
                            nullptr);
        store_tile<T>(kr, vr, smem);
    }
    __syncthreads();
    // is the lane's row one of the global positions?  (binary search of the
    // sorted list; the same number of steps on every lane)
    bool row_glob = false;
    if constexpr (GLOB) {
        int pos = 0;
        for (int w = 1 << (31 - __builtin_clz(p.n_global)); w > 0; w >>= 1)
            if (pos + w <= p.n_global && gpos_lds[pos + w - 1] < qpos) pos += w;
        row_glob = qpos >= 0 && pos < p.n_global && gpos_lds[pos] == qpos;
    }

    const int tr_off = tr_row(lane) * T::KP + tr_col(lane);
    // Band tiles, then (GLOB) the gathered global-key tiles in a copy of the
    // step of their own, so that the band loop keeps only the band's masks
    // and row loads.  The band loop does not prefetch the first gathered
    // tile; its step loads it.
    const int n_main = GLOB ? min(ks.n_band_tiles, ks.n_tiles) : ks.n_tiles;
    auto step = [&](const int j, auto gath_tag) {
        constexpr bool GATH = decltype(gath_tag)::value;
        constexpr bool kBandLoads = GLOB && !GATH;
        const int st = j & 1;
        const bool has_next = j + 1 < (GATH ? ks.n_tiles : n_main);
        if constexpr (GATH) {
            if (j == n_main) {
                load_tile<T, false>(kr, vr, kbase, vbase, kbase, vbase, rowstride, ks, p, j,
                                    gk_lds[st], gpos_ptr);
                store_tile<T>(kr, vr, smem + st * T::STAGE);
                __syncthreads();
            }
        }
        const int kt0 = ks.k_lo + j * BN;
        const int kt1 = kt0 + BN - 1;
        const bool skip =
            !GATH && (w_first > w_last || kt0 > w_last + p.wr || kt1 < w_first - p.wl);
        const bool need_mask =
            GATH || !(kt0 >= w_last - p.wl && kt1 <= w_first + p.wr && kt1 <= ks.k_hi);
        const unsigned short* Ks = smem + st * T::STAGE;
        const unsigned short* Vs = Ks + T::K_ELEMS;
        if (skip && has_next)
            load_tile<T, kBandLoads>(kr, vr, kbase, vbase, kbase, vbase, rowstride, ks, p, j + 1,
                                     gk_lds[st ^ 1], gpos_ptr);
        if (!skip) {
            // one 32-key block at a time: S^T = K Q^T and dP^T = V dout^T for
            // its keys, then dS^T and dq^T += K^T dS^T over its two 16-key
            // steps (half the score registers live at once)
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int kc = 0; kc < KC; kc++) {
                    const bf16x8 ka =
                        *(const bf16x8*)(Ks + (kb * 32 + l32) * T::KP + kc * 16 + half * 8);
                    const bf16x8 va =
                        *(const bf16x8*)(Vs + (kb * 32 + l32) * T::VP + kc * 16 + half * 8);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[kc], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, greg[kc], dp, 0, 0, 0);
                }
                // the next tile's loads go out after the first block's score MFMAs
                // (issued before them, the compiler would wait for the loads
                // ahead of the MFMAs, whose results may reuse their address
                // registers)
                if (kb == 0 && has_next)
                    load_tile<T, kBandLoads>(kr, vr, kbase, vbase, kbase, vbase, rowstride, ks,
                                             p, j + 1, gk_lds[st ^ 1], gpos_ptr);
                if (GATH) {
                    // gathered global keys (position g, residue coordinate r of
                    // g): hidden when padding (g < 0), in the row's band, after
                    // a causal row, or for every key when the row is global
                    const int* gk = gk_lds[st];
                    const int span = p.wl + p.wr;
                    const int causal_mask = p.causal ? -1 : 0;
                    const int row_bad = row_glob ? -1 : 0;
#pragma unroll
                    for (int e4 = 0; e4 < 4; e4++) {
                        const int4 g4 = *(const int4*)(gk + kb * 32 + e4 * 8 + half * 4);
                        const int4 r4 = *(const int4*)(gk + BN + kb * 32 + e4 * 8 + half * 4);
                        const int gv[4] = {g4.x, g4.y, g4.z, g4.w};
                        const int rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                        for (int e3 = 0; e3 < 4; e3++) {
                            const int x = rv[e3] - qres + p.wl;
                            const int inband = ~(x | (span - x)) >> 31;
                            const int future = causal_mask & ((qpos - gv[e3]) >> 31);
                            const int bad = (gv[e3] >> 31) | inband | future | row_bad;
                            s[e4 * 4 + e3] += __builtin_bit_cast(float, bad & 0xff800000);
                        }
                    }
                } else if (need_mask) {
                    // the forward's band edge masks (x = key - query + wl in
                    // [0, wl + wr], key <= k_hi): the lane's valid offsets form
                    // one interval [lo, hi] (an empty one moved past the tile),
                    // one unsigned range compare and a select per element
                    const int base = kt0 + half * 4 - qres + p.wl;
                    int lo = -base;
                    int hi = min(p.wl + p.wr - base, ks.k_hi - kt0 - half * 4);
                    if (hi < lo) lo = hi = 1 << 20;
                    const unsigned span = (unsigned)(hi - lo);
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int ko = kb * 32 + (e >> 2) * 8 + (e & 3);
                        if ((unsigned)(ko - lo) > span) s[e] = -INFINITY;
                    }
                }
                // dS^T = P^T (dP^T - delta), bf16, in the slot order of the K^T
                // reads; then dq^T += K^T dS^T over this block's 16-key steps
#pragma unroll
                for (int t = 2 * kb; t < 2 * kb + 2; t++) {
                    bf16x8 ds;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const int ei = (t & 1) * 8 + slot_elem(e);
                        const float pe = fast_exp2(__builtin_fmaf(s[ei], c, -lse2));
                        ds[e] = (__bf16)(pe * (dp[ei] - dlt));
                    }
#pragma unroll
                    for (int db = 0; db < DB; db++) {
                        const unsigned short* kp = Ks + tr_off + t * 16 * T::KP + tr_block_col(db);
                        const i16x4 lo = lds_read_tr16(kp);
                        const i16x4 hi = lds_read_tr16(kp + kTrHi * T::KP);
                        const bf16x8 ka = __builtin_bit_cast(
                            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                        dqacc[db] =
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, ds, dqacc[db], 0, 0, 0);
                    }
                }
            }
        }
        SWA_DEBUG_BARRIER();   // every wave's reads of this stage are done
        if (has_next) store_tile<T>(kr, vr, smem + (st ^ 1) * T::STAGE);
        __syncthreads();
    };
    for (int j = 0; j < n_main; j++) step(j, std::false_type{});
    if constexpr (GLOB)
        for (int j = n_main; j < ks.n_tiles; j++) step(j, std::true_type{});

    if (qpos < 0) return;
    SWA_DCHECK(qpos < p.N && hq < p.Hq);
    // dq^T block: element (db, jq*4 + e) is dim acc_dim(db, jq, half) + e of query l32
    __bf16* op = (__bf16*)bp.dq + (((size_t)b * p.N + qpos) * p.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int jq = 0; jq < 4; jq++) {
            bf16x4 o4;
#pragma unroll
            for (int e = 0; e < 4; e++) o4[e] = (__bf16)(dqacc[db][jq * 4 + e] * bp.scale);
            *(bf16x4*)(op + acc_dim(db, jq, half)) = o4;
        }
}

// ---- 3. dk, dv: key-major ------------------------------------------------------------
constexpr int BK = 128;   // keys per workgroup (four waves of 32)
constexpr int BQ = 64;    // query rows per staged tile

template <int D>
struct QTileCfg {
    static constexpr int QP = D + 8;                  // row pitch (bf16) of the Q and dout tiles
    static constexpr int ELEMS = BQ * QP;
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int PER_THREAD = BQ * CPR / 256;
    static constexpr int ROW_STEP = 256 / CPR;
};

// Fragments of one 16-deep k-step of S = Q K^T and dP = dout V^T: the two
// 32-query row blocks of Q and of dout (A operands, 16 bytes per lane).
template <int D>
struct ScoreFrag {
    bf16x8 q[2], g[2];
};
template <int D>
__device__ __forceinline__ ScoreFrag<D> read_score_frag(const unsigned short* Qs, int kc,
                                                        int l32, int half) {
    using Q = QTileCfg<D>;
    ScoreFrag<D> f;
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
        const int off = (rb * 32 + l32) * Q::QP + kc * 16 + half * 8;
        f.q[rb] = *(const bf16x8*)(Qs + off);
        f.g[rb] = *(const bf16x8*)(Qs + Q::ELEMS + off);
    }
    return f;
}

// Transposed fragments of one 16-query step t: dout^T and Q^T for every
// 32-row block of the head dimension.
template <int D>
struct TrFrag {
    bf16x8 g[D / 32], q[D / 32];
};
template <int D>
__device__ __forceinline__ TrFrag<D> read_tr_frag(const unsigned short* Qs, int tr_off, int t) {
    using Q = QTileCfg<D>;
    TrFrag<D> f;
#pragma unroll
    for (int db = 0; db < D / 32; db++) {
        const int off = tr_off + t * 16 * Q::QP + tr_block_col(db);
        const unsigned short* gp = Qs + Q::ELEMS + off;
        const unsigned short* qp = Qs + off;
        const i16x4 glo = lds_read_tr16(gp), ghi = lds_read_tr16(gp + kTrHi * Q::QP);
        const i16x4 qlo = lds_read_tr16(qp), qhi = lds_read_tr16(qp + kTrHi * Q::QP);
        f.g[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7));
        f.q[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    return f;
}

// At D = 128 a wave's accumulators (dk, dv: 128 registers), K and V (64) and
// two steps' scores (128) need one wave per SIMD, and the wave overlaps its
// own work (the next step's scores beside this step's exponentials).  At D =
// 64 one step's scores fit beside the rest in 256 registers: two waves share
// each SIMD and overlap each other, and a step runs in plain order.
template <int D>
constexpr bool kDkdvPipelined = D == 128;

template <int D>
__global__ __launch_bounds__(256, (kDkdvPipelined<D> ? 1 : 2))
void bwd_dkdv_bf16_kernel(const BwdParams bp) {
    using Q = QTileCfg<D>;
    const FwdParams& p = bp.f;
    constexpr int KC = D / 16;
    constexpr int DB = D / 32;
    // Three LDS stages.  During step st tile st + 2 is staged.  Pipelined
    // (D = 128): the dk/dv products read tile st and the scores of step st + 1
    // read tile st + 1, so the next step's score MFMAs run beside this step's
    // exponentials.  Plain order (D = 64): step st reads tile st only, and
    // the loads of tile st + 2 have two steps to arrive.
    constexpr int NS = 3;

    // per stage: Q tile, dout tile, lse2[BQ], delta[BQ]
    __shared__ __attribute__((aligned(16))) unsigned short qsm[NS][2 * Q::ELEMS];
    __shared__ __attribute__((aligned(16))) float rsm[NS][2 * BQ];
    // D = 64 with global tokens: after the band's steps, gathered steps stage
    // the global rows (64 to a tile, for every query head of the group) and
    // add their pairs with this block's keys outside their band (causal: not
    // after the row), the global-row dk/dv pairs.  Per stage the rows'
    // positions (-1: padding) and residue coordinates (this block's class,
    // else a value no window reaches) feed the masks.
    constexpr bool kGathRows = !kDkdvPipelined<D>;
    __shared__ int gpos_lds[kGathRows ? SWA_MAX_GLOBAL : 1];
    __shared__ __attribute__((aligned(16))) int rpos[kGathRows ? NS : 1][2 * BQ];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l32 = lane & 31;
    const int half = lane >> 5;

    // work item: (b, kv head, residue class, key block); the longest blocks of
    // a slab first.  A key block's query rows run off the end of the sequence
    // when the window reaches further left than right (causal): those blocks
    // are the short ones, so then the slab goes from the first block to the
    // last (the mirror of the forward's order).  Workgroups that start
    // together also stay in step, and read the same query tiles while L2
    // still holds them.
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
    const int kb0 = kt * BK;
    const int kb1 = min(kb0 + BK - 1, Nr - 1);
    const int wk0 = kb0 + wave * 32;               // this wave's first key
    const int wk1 = min(wk0 + 31, kb1);
    // query rows whose windows reach the block: i - wl <= j <= i + wr
    const int q_lo = max(0, kb0 - p.wr);
    const int q_hi = min(Nr - 1, kb1 + p.wl);
    const int n_qt = (q_hi - q_lo + BQ) / BQ;
    const int n_band_steps = n_qt * p.group;       // (query head, query tile) pairs
    const int n_gt = kGathRows && p.n_global > 0 ? (p.n_global + BQ - 1) / BQ : 0;
    const int n_steps = n_band_steps + n_gt * p.group;   // then (head, gathered tile)

    // the lane's key as the B operand of S = Q K^T and dP = dout V^T
    const int key = wk0 + l32;
    const bool key_ok = key <= kb1;
    const int kpos = r + min(key, kb1) * p.dil;
    bf16x8 kreg[KC], vreg[KC];
    {
        const size_t ko = (((size_t)b * p.N + kpos) * p.Hkv + kvh) * D + half * 8;
        const __bf16* kp = (const __bf16*)p.k + ko;
        const __bf16* vp = (const __bf16*)p.v + ko;
        const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            kreg[kc] = key_ok ? *(const bf16x8*)(kp + kc * 16) : z;
            vreg[kc] = key_ok ? *(const bf16x8*)(vp + kc * 16) : z;
        }
    }
    f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) dkacc[db] = dvacc[db] = f32x16{};
    const float c = p.scale_log2;
    const int span = p.wl + p.wr;

    // staging of step st (clamped to the last step, so a load past the end
    // re-reads that step's rows): query head st / n_qt, tile st % n_qt.  Rows
    // past q_hi take row q_hi's values: the element masks of such a tile (it
    // always takes them) zero P and dS there, and the values are finite.
    u32x4 qr[Q::PER_THREAD], gr[Q::PER_THREAD];
    float rl = 0.f;
    int rp_pos = -1, rp_res = kFarAway;   // gathered steps: the row of thread t < BQ
    if (n_gt > 0) {
        for (int i = threadIdx.x; i < p.n_global; i += 256) gpos_lds[i] = p.gpos[i];
        __syncthreads();
    }
    auto load_step = [&](int st) {
        st = min(st, n_steps - 1);
        const bool gth = kGathRows && st >= n_band_steps;   // uniform
        int hq, q0;
        if (!gth) {
            hq = kvh * p.group + st / n_qt;
            q0 = q_lo + (st % n_qt) * BQ;
        } else {
            // q0: index of the tile's first row in the global list
            hq = kvh * p.group + (st - n_band_steps) / n_gt;
            q0 = ((st - n_band_steps) % n_gt) * BQ;
        }
        // absolute position of tile row rr (band rows past q_hi repeat q_hi;
        // gathered rows past the list repeat its last entry)
        auto row_pos = [&](int rr) {
            return gth ? gpos_lds[min(q0 + rr, p.n_global - 1)]
                       : r + min(q0 + rr, q_hi) * p.dil;
        };
        if constexpr (kGathRows) {
            const int rr = threadIdx.x & (BQ - 1);
            rp_pos = gth && q0 + rr < p.n_global ? gpos_lds[q0 + rr] : -1;
            rp_res = rp_pos >= 0 && rp_pos % p.dil == r ? rp_pos / p.dil : kFarAway;
        }
        // lse for threads 0..63, delta for 64..127, one row each (later lanes
        // read a row again and drop it, so the load needs no branch).  It is
        // issued before the tile rows and used only when stored (lse scaled to
        // base 2 there): any wait the compiler places around it, for a register
        // kept in scratch say, then cannot include the tile loads, which would
        // stall the step for their whole latency.
        const int row0 = threadIdx.x / Q::CPR, cc = threadIdx.x % Q::CPR;
        if constexpr (!kGathRows) {
            {
                const int qrow = min(q0 + (int)(threadIdx.x & (BQ - 1)), q_hi);
                const size_t li = ((size_t)b * p.Hq + hq) * p.N + r + (size_t)qrow * p.dil;
                rl = *((threadIdx.x < BQ ? p.lse : bp.delta) + li);
            }
#pragma unroll
            for (int u = 0; u < Q::PER_THREAD; u++) {
                const int qrow = min(q0 + row0 + u * Q::ROW_STEP, q_hi);
                SWA_DCHECK(qrow >= 0 && r + qrow * p.dil < p.N && hq < p.Hq);
                const size_t off =
                    (((size_t)b * p.N + r + (size_t)qrow * p.dil) * p.Hq + hq) * D + cc * 8;
                qr[u] = *(const u32x4*)((const __bf16*)p.q + off);
                gr[u] = *(const u32x4*)((const __bf16*)bp.dout + off);
            }
            return;
        }
        {
            const int pos = row_pos((int)(threadIdx.x & (BQ - 1)));
            const size_t li = ((size_t)b * p.Hq + hq) * p.N + pos;
            rl = *((threadIdx.x < BQ ? p.lse : bp.delta) + li);
        }
#pragma unroll
        for (int u = 0; u < Q::PER_THREAD; u++) {
            const int pos = row_pos(row0 + u * Q::ROW_STEP);
            SWA_DCHECK(pos >= 0 && pos < p.N && hq < p.Hq);
            const size_t off = (((size_t)b * p.N + pos) * p.Hq + hq) * D + cc * 8;
            qr[u] = *(const u32x4*)((const __bf16*)p.q + off);
            gr[u] = *(const u32x4*)((const __bf16*)bp.dout + off);
        }
    };
    auto store_step = [&](int stage) {
        const int row0 = threadIdx.x / Q::CPR, cc = threadIdx.x % Q::CPR;
        unsigned short* qs = qsm[stage];
        unsigned short* gs = qs + Q::ELEMS;
#pragma unroll
        for (int u = 0; u < Q::PER_THREAD; u++) {
            const int rw = row0 + u * Q::ROW_STEP;
            SWA_DCHECK(rw < BQ && stage < NS);
            *(u32x4*)(qs + rw * Q::QP + cc * 8) = qr[u];
            *(u32x4*)(gs + rw * Q::QP + cc * 8) = gr[u];
        }
        if (threadIdx.x < 2 * BQ) rsm[stage][threadIdx.x] = threadIdx.x < BQ ? rl * kLog2e : rl;
        if constexpr (kGathRows)
            if (threadIdx.x < BQ) {
                rpos[stage][threadIdx.x] = rp_pos;
                rpos[stage][BQ + threadIdx.x] = rp_res;
            }
    };

    const int tr_off = tr_row(lane) * Q::QP + tr_col(lane);
    f32x16 sc[2][2], dpc[2][2];   // scores and dP of two consecutive steps
    // one k-step of S and dP into the set (s, dp)
    auto scores = [&](f32x16 (&s)[2], f32x16 (&dp)[2], int kc, const ScoreFrag<D>& f) {
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.q[rb], kreg[kc], s[rb], 0, 0, 0);
            dp[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.g[rb], vreg[kc], dp[rb], 0, 0, 0);
        }
    };
    if (n_steps > 0) {   // uniform over the workgroup
        load_step(0);
        store_step(0);
        load_step(1);
        store_step(1);
        __syncthreads();
        if constexpr (kDkdvPipelined<D>) {
            sc[0][0] = sc[0][1] = dpc[0][0] = dpc[0][1] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < KC; kc++)
                scores(sc[0], dpc[0], kc, read_score_frag<D>(qsm[0], kc, l32, half));
        }
    }

    // One step: tile st in stage st % NS, its scores in set PAR.  The source
    // order below is the issue order (the fences keep the compiler from
    // regrouping it): the next step's score MFMAs, each k-step's fragments read
    // one k-step ahead, with this step's P and dS computed between them; then
    // the dk/dv MFMAs, each 16-query step's transposed fragments read one step
    // ahead.
    auto step = [&](int st, auto par_tag) {
        constexpr int PAR = decltype(par_tag)::value;
        const int stage = st % NS;
        const int stage_next = (st + 1) % NS;
        const int stage_store = (st + 2) % NS;
        const int q0 = q_lo + (st % n_qt) * BQ;
        const int q1 = q0 + BQ - 1;
        // wave-uniform: every pair of this wave's keys with these queries valid?
        const bool need_mask = !(q0 >= wk1 - p.wr && q1 <= wk0 + p.wl && q1 <= q_hi &&
                                 wk0 + 31 <= kb1);
        f32x16 (&s)[2] = sc[PAR];
        f32x16 (&dp)[2] = dpc[PAR];
        if (need_mask) {
            // element (rb, e) is query q0 + rb*32 + (e>>2)*8 + half*4 + (e&3) and key
            // `key`: valid when query - key + wr lies in [0, wl + wr], the query
            // is <= q_hi and the key <= kb1
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                const int base = q0 + rb * 32 + half * 4 - key + p.wr;
                const int qlim = q_hi - (q0 + rb * 32 + half * 4);
                const int kbad = kb1 - key;
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int ro = (e >> 2) * 8 + (e & 3);
                    const int bad = ((base + ro) | (span - base - ro) | (qlim - ro) | kbad) >> 31;
                    s[rb][e] += __builtin_bit_cast(float, bad & 0xff800000);
                }
            }
        }
        // next tile's rows into registers (stored at the end of the step).  At
        // D = 128 the PAR = 0 copy issues them after phase 1 instead: at its
        // score-phase register peak the compiler would otherwise move the
        // fresh loads to other registers and wait for them on the spot.
        constexpr bool late_load = D == 128 && PAR == 0;
        if (!late_load) load_step(st + 2);
        const unsigned short* Qs = qsm[stage];
        const unsigned short* Qn = qsm[stage_next];
        const float* lse2 = rsm[stage];
        const float* dlt = lse2 + BQ;
        f32x16 (&sn)[2] = sc[PAR ^ 1];
        f32x16 (&dpn)[2] = dpc[PAR ^ 1];
        sn[0] = sn[1] = dpn[0] = dpn[1] = f32x16{};

        // phase 1: scores of step st + 1 (past the last step they read a stale
        // stage and are never used) beside P and dS of step st, half a
        // 16-query step per k-step
        bf16x8 pb[4], dsb[4];
        ScoreFrag<D> fr[2];
        fr[0] = read_score_frag<D>(Qn, 0, l32, half);
        f32x4 lr[4];   // lse2 rows 0..3 and 8..11 of the step, then delta's
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            __builtin_amdgcn_sched_barrier(0);
            if (kc + 1 < KC) fr[(kc + 1) & 1] = read_score_frag<D>(Qn, kc + 1, l32, half);
            // this k-step's share of P and dS: elements g0 .. g0 + PER - 1 of the
            // step's 32 (16-query step t, slots e0 ..)
            constexpr int PER = 32 / KC;
            const int g0 = kc * PER;
            const int t = g0 / 8;
            const int e0 = g0 % 8;
            const int rowb = (t >> 1) * 32 + (t & 1) * 16 + half * 4;
            if (e0 == 0) {
                lr[0] = *(const f32x4*)(lse2 + rowb);
                lr[1] = *(const f32x4*)(lse2 + rowb + 8);
                lr[2] = *(const f32x4*)(dlt + rowb);
                lr[3] = *(const f32x4*)(dlt + rowb + 8);
            }
            scores(sn, dpn, kc, fr[kc & 1]);
#pragma unroll
            for (int i = 0; i < PER; i++) {
                const int e = e0 + i;
                const int el = slot_elem(e);          // row rowb + (el>>2)*8 + (el&3)
                const int ei = (t & 1) * 8 + el;
                const float l2 = lr[el >> 2][el & 3];
                const float dl = lr[2 + (el >> 2)][el & 3];
                const float pe = fast_exp2(__builtin_fmaf(s[t >> 1][ei], c, -l2));
                pb[t][e] = (__bf16)pe;
                dsb[t][e] = (__bf16)(pe * (dp[t >> 1][ei] - dl));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (late_load) load_step(st + 2);

        // phase 2: dv^T += dout^T P and dk^T += Q^T dS over four 16-query steps
        TrFrag<D> tf[2];
        tf[0] = read_tr_frag<D>(Qs, tr_off, 0);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            __builtin_amdgcn_sched_barrier(0);
            if (t + 1 < 4) tf[(t + 1) & 1] = read_tr_frag<D>(Qs, tr_off, t + 1);
#pragma unroll
            for (int db = 0; db < DB; db++) {
                dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[t & 1].g[db], pb[t],
                                                                    dvacc[db], 0, 0, 0);
                dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[t & 1].q[db], dsb[t],
                                                                    dkacc[db], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // stage (st + 2) % NS held tile st - 1, which every wave finished before
        // the previous barrier
        SWA_DEBUG_BARRIER();
        store_step(stage_store);
        __syncthreads();
    };
    // One step in plain order (two waves per SIMD): tile st + 2's rows into
    // registers, this step's S and dP, their masks, P and dS, the dk/dv
    // MFMAs, then the store of tile st + 2 into the stage tile st - 1 held.
    auto step_plain = [&](int st) {
        const int stage = st % NS;
        const int stage_store = (st + 2) % NS;
        const int q0 = q_lo + (st % n_qt) * BQ;
        const int q1 = q0 + BQ - 1;
        const bool need_mask = !(q0 >= wk1 - p.wr && q1 <= wk0 + p.wl && q1 <= q_hi &&
                                 wk0 + 31 <= kb1);
        load_step(st + 2);
        const unsigned short* Qs = qsm[stage];
        const float* lse2 = rsm[stage];
        const float* dlt = lse2 + BQ;
        f32x16 s[2], dp[2];
        s[0] = s[1] = dp[0] = dp[1] = f32x16{};
        ScoreFrag<D> fr[2];
        fr[0] = read_score_frag<D>(Qs, 0, l32, half);
#pragma unroll
        for (int kc = 0; kc < KC; kc++) {
            if (kc + 1 < KC) fr[(kc + 1) & 1] = read_score_frag<D>(Qs, kc + 1, l32, half);
            scores(s, dp, kc, fr[kc & 1]);
        }
        if (kGathRows && st >= n_band_steps) {
            // gathered global rows: hidden when padding (position < 0), when
            // the key lies in the row's band (x = row - key + wr in [0, wl +
            // wr], residue coordinates of this class), after a causal row, or
            // past kb1
            const int* rp = rpos[stage];
            const int causal_mask = p.causal ? -1 : 0;
            const int kbad = (kb1 - key) >> 31;
#pragma unroll
            for (int rb = 0; rb < 2; rb++)
#pragma unroll
                for (int e4 = 0; e4 < 4; e4++) {
                    const int4 p4 = *(const int4*)(rp + rb * 32 + e4 * 8 + half * 4);
                    const int4 r4 = *(const int4*)(rp + BQ + rb * 32 + e4 * 8 + half * 4);
                    const int pv[4] = {p4.x, p4.y, p4.z, p4.w};
                    const int rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                    for (int e3 = 0; e3 < 4; e3++) {
                        const int x = rv[e3] - key + p.wr;
                        const int inband = ~(x | (span - x)) >> 31;
                        const int future = causal_mask & ((pv[e3] - kpos) >> 31);
                        const int bad = (pv[e3] >> 31) | inband | future | kbad;
                        s[rb][e4 * 4 + e3] += __builtin_bit_cast(float, bad & 0xff800000);
                    }
                }
        } else if (need_mask) {
            // the band: query - key + wr in [0, wl + wr], query <= q_hi, key <=
            // kb1 (the pipelined step keeps its sign-bit form of the same test:
            // there this form took more registers and measured slower)
            // The lane's valid query offsets qo (from q0 + half * 4) form one
            // interval [lo, hi] (an empty one moved past the tile): one
            // unsigned range compare and a select per element.
            {
                const int q_base = q0 + half * 4;
                int lo = key - p.wr - q_base;
                int hi = min(lo + span, q_hi - q_base);
                if (key > kb1 || hi < lo) lo = hi = 1 << 20;
                const unsigned width = (unsigned)(hi - lo);
#pragma unroll
                for (int rb = 0; rb < 2; rb++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int qo = rb * 32 + (e >> 2) * 8 + (e & 3);
                        if ((unsigned)(qo - lo) > width) s[rb][e] = -INFINITY;
                    }
            }
        }
        // P and dS of the step's four 16-query steps (8 elements each per lane)
        bf16x8 pb[4], dsb[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int rowb = (t >> 1) * 32 + (t & 1) * 16 + half * 4;
            f32x4 lr[4];
            lr[0] = *(const f32x4*)(lse2 + rowb);
            lr[1] = *(const f32x4*)(lse2 + rowb + 8);
            lr[2] = *(const f32x4*)(dlt + rowb);
            lr[3] = *(const f32x4*)(dlt + rowb + 8);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int el = slot_elem(e);
                const int ei = (t & 1) * 8 + el;
                const float pe = fast_exp2(__builtin_fmaf(s[t >> 1][ei], c, -lr[el >> 2][el & 3]));
                pb[t][e] = (__bf16)pe;
                dsb[t][e] = (__bf16)(pe * (dp[t >> 1][ei] - lr[2 + (el >> 2)][el & 3]));
            }
        }
        // dv^T += dout^T P and dk^T += Q^T dS over the four 16-query steps
        TrFrag<D> tf[2];
        tf[0] = read_tr_frag<D>(Qs, tr_off, 0);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            if (t + 1 < 4) tf[(t + 1) & 1] = read_tr_frag<D>(Qs, tr_off, t + 1);
#pragma unroll
            for (int db = 0; db < DB; db++) {
                dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[t & 1].g[db], pb[t],
                                                                    dvacc[db], 0, 0, 0);
                dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[t & 1].q[db], dsb[t],
                                                                    dkacc[db], 0, 0, 0);
            }
        }
        SWA_DEBUG_BARRIER();
        store_step(stage_store);
        __syncthreads();
    };
    if constexpr (kDkdvPipelined<D>) {
        for (int st = 0; st < n_steps; st += 2) {
            step(st, std::integral_constant<int, 0>{});
            if (st + 1 < n_steps) step(st + 1, std::integral_constant<int, 1>{});
        }
    } else {
        for (int st = 0; st < n_steps; st++) step_plain(st);
    }

    if (!key_ok) return;
    SWA_DCHECK(kpos >= 0 && kpos < p.N);
    const size_t ko = (((size_t)b * p.N + kpos) * p.Hkv + kvh) * D;
    __bf16* dkp = (__bf16*)bp.dk + ko;
    __bf16* dvp = (__bf16*)bp.dv + ko;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int jq = 0; jq < 4; jq++) {
            bf16x4 k4, v4;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                k4[e] = (__bf16)(dkacc[db][jq * 4 + e] * bp.scale);
                v4[e] = (__bf16)dvacc[db][jq * 4 + e];
            }
            *(bf16x4*)(dkp + acc_dim(db, jq, half)) = k4;
            *(bf16x4*)(dvp + acc_dim(db, jq, half)) = v4;
        }
}

template <int D, typename T>
hipError_t launch_delta(const BwdParams& p, hipStream_t s) {
    const int64_t rows = (int64_t)p.f.B * p.f.N * p.f.Hq;
    const int64_t dblocks = (rows * (D / 8) + 255) / 256;
    if (dblocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_delta_kernel<D, T>), dim3((unsigned)dblocks), dim3(256), 0, s,
                       (const T*)p.out, (const T*)p.dout, p.delta, p.f.Hq, p.f.N, rows);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdParams& p, hipStream_t s) {
    if (p.f.n_global > 0)
        hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, 4, true>), dim3(p.f.n_blocks), dim3(256), 0, s,
                           p);
    else
        hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, 4, false>), dim3(p.f.n_blocks), dim3(256), 0,
                           s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D>), dim3(p.k_blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

FwdShape bwd_bf16_dq_shape(int group) {
    // four waves: the heads of a GQA group that share the K/V tiles, times rows
    const int hpw = group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
    const int rows = (4 / hpw) * 32;
    return FwdShape{hpw, rows, rows};
}

int bwd_bf16_dkdv_keys() { return BK; }

hipError_t launch_bwd_bf16(const BwdParams& p, int D, hipStream_t s) {
    return D == 128 ? launch_d<128>(p, s) : launch_d<64>(p, s);
}

// float32 only: the bf16 dq pass computes delta for its rows itself.
hipError_t launch_bwd_delta(const BwdParams& p, int D, hipStream_t s) {
    return D == 128 ? launch_delta<128, float>(p, s) : launch_delta<64, float>(p, s);
}

#ifdef SWA_DEBUG
SWA_DEBUG_COUNTER_READER(debug_counter_bwd_bf16)
#endif

}  // namespace swa
