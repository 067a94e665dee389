// fwd_pp.hip -- sliding-window attention forward, bf16, D = 128, band only:
// eight waves in two groups that run half a step apart.
//
// What is computed is exactly what the single-phase forward kernel computes
// (the same tiles, masks, lazily rescaled online softmax and bf16-rounded
// weights; aiqz.cc "Sliding window attention: Mistral", the band of section
// "sliding window"; bmjup.com "Sliding window attention", section 3 for the
// O(n*W) walk).  Only the order of the work differs.
//
// Per K/V tile a wave has a matrix phase (P V of the previous tile, then
// S^T = K Q^T of this tile: 32 MFMAs of 32x32x16) and a vector phase (masks,
// running max, exponentials, row sums).  With one barrier per tile both waves
// that share a SIMD are in the same phase at the same time, and the matrix
// core idles while they both run the softmax.  Here waves 0-3 (group A) and
// 4-7 (group B) -- one of each on every SIMD -- are offset by one phase, with
// a barrier between phases: while one group runs its MFMAs the other runs its
// softmax on the same SIMD.  A's phases are 2t (matrix, tile t) and 2t+1
// (vector); B's are 2t+1 and 2t+2.  Every wave passes 2n + 1 barriers for n
// tiles: B one extra before its first phase, A one after its last.
//
// K and V tiles go from global memory straight into LDS (global_load_lds:
// no staging registers, no LDS stores), three slots per tensor.  Group A
// loads K_{t+2} at the start of its vector phase 2t+1, into the slot of
// K_{t-1} (last read in phase 2t-1); group B loads V_{t+2} at the start of its
// vector phase 2t+2, into the slot of V_{t-1} (last read in phase 2t+1).  Each
// wave waits for its loads of a tile at the end of its next vector phase,
// before the barrier after which the tile is first read (phase 2t+4 for K,
// 2t+6 for V): a load has three phases to arrive.  The compiler does not see
// these loads (they are issued in inline assembly, so that it does not make
// every later LDS read wait for them); the waits are explicit.
//
// LDS layout: a load writes 1 KB, four 256-byte rows, per instruction, so
// rows are stored in groups of four, each group followed by 64 bytes of
// padding; the 16-byte chunk c of row 4g + q is stored at position c ^ f(q)
// of its row, f(q) = q for K and 4q for V.  A K fragment read serves 16 lanes
// per LDS cycle, 16 consecutive rows at one chunk: the padding moves each of
// the four groups 16 banks on, and c ^ q spreads the four rows of a group
// over the four positions of an aligned quad.  A transposing V read serves
// 32 lanes, 4 rows of one group x 4 consecutive chunks: c ^ 4q gives each row
// its own quad.  Both are free of bank conflicts, and both keep the offsets
// that vary across a wave's reads (k-step, key step) immediate: K needs one
// base address for even and one for odd k-steps, V one per 32-column block.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fwd_common.h"
#include "swa_kernels.h"
#include "tile_common.h"

namespace swa {
namespace {

constexpr int D = 128;
constexpr int KC = D / 16;           // 16-deep k-steps of K Q^T
constexpr int DB = D / 32;           // 32-row blocks of O^T
constexpr int ROW = D;                 // row length (bf16 elements)
constexpr int GRP = 4 * ROW + 32;      // four rows and 64 bytes of padding
constexpr int SLOT = BN / 4 * GRP;     // one tile of one tensor
constexpr int NSLOT = 3;
constexpr int LOADS = BN / 4 / 4;      // 1 KB loads per wave per tile (one group each)
static_assert(LOADS == 4, "the wait counts below assume four loads per tile");

// chunk position factor: K stores chunk c of row 4g + q at c ^ q, V at c ^ 4q
template <bool V>
__device__ __forceinline__ int chunk_xor(int q) { return V ? 4 * q : q; }

// 16 bytes per lane from global memory to LDS at m0 + 16 * lane (one wait
// state between the write of m0 and the load that reads it): from a per-lane
// address, or from a wave-uniform base plus a per-lane 32-bit byte offset
// (m0 is declared clobbered: the compiler keeps nothing there across them)
__device__ __forceinline__ void load_lds_x4(const void* src, unsigned lds_byte) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_byte), "v"(src)
                 : "memory", "m0");
}
__device__ __forceinline__ void load_lds_x4(const void* base, unsigned off, unsigned lds_byte) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_byte), "v"(off), "s"(base)
                 : "memory", "m0");
}

__global__ __launch_bounds__(512, 1) void swa_fwd_pp_kernel(const FwdParams p) {
    __shared__ __attribute__((aligned(1024))) unsigned short k_lds[NSLOT * SLOT];
    __shared__ __attribute__((aligned(1024))) unsigned short v_lds[NSLOT * SLOT];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;          // 0: A (loads K), 1: B (loads V)
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

    // ---- query rows of this wave (B operand of S^T = K Q^T) ----------------
    const int qres = wave_row0 + l32;
    const int qpos = qres < ks.Nr ? ks.r + qres * ks.dil : -1;
    bf16x8 qreg[KC];
    {
        const __bf16* qp =
            (const __bf16*)p.q + (((size_t)b * p.N + max(qpos, 0)) * p.Hq + hq) * D + half * 8;
#pragma unroll
        for (int kc = 0; kc < KC; kc++)
            qreg[kc] = qpos >= 0 ? *(const bf16x8*)(qp + kc * 16)
                                 : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    const int w_first = wave_row0;
    const int w_last = min(wave_row0 + 31, ks.Nr - 1);

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] = f32x16{};
    float m_run = kEmptyMax;
    const float c = p.scale_log2;
    const __bf16 one = (__bf16)1.0f;
    const bf16x2 ones = {one, one};

    // ---- tile loads --------------------------------------------------------------
    // Load u of a wave covers rows row0 + 4u .. +3 of the tile: lane l writes
    // position l & 15 of row row0 + 4u + (l >> 4), so it fetches the chunk
    // stored there.  Rows past k_hi (last tile only, always element-masked)
    // repeat row k_hi.
    const unsigned k_lds_b = (unsigned)(size_t)(__attribute__((address_space(3))) void*)k_lds;
    const unsigned v_lds_b = (unsigned)(size_t)(__attribute__((address_space(3))) void*)v_lds;
    auto load_tile_rows = [&](const __bf16* base, unsigned lds_b, bool is_v, int t, int row0) {
        const unsigned slot_b = lds_b + (unsigned)((t % NSLOT) * SLOT * 2);
        // (lane values from an opaque copy of the thread index: see below)
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
#pragma unroll
        for (int u = 0; u < LOADS; u++) {
            const int q = (tid >> 4) & 3;
            const int r = row0 + 4 * u + q;
            const int chunk = (tid & 15) ^ (is_v ? chunk_xor<true>(q) : chunk_xor<false>(q));
            const int kk = min(ks.k_lo + t * BN + r, ks.k_hi);
            SWA_DCHECK(kk >= 0 && ks.r + kk * ks.dil < p.N && chunk < 16);
            SWA_DCHECK(slot_b + (row0 / 4 + u) * GRP * 2 + 1024 <= lds_b + NSLOT * SLOT * 2);
            const __bf16* src = base + (size_t)(ks.r + kk * ks.dil) * rowstride + chunk * 8;
            load_lds_x4(src, slot_b + (unsigned)((row0 / 4 + u) * GRP * 2));
        }
    };
    // The same loads for a tile that lies inside [k_lo, k_hi] (every tile but
    // the last): a wave-uniform row base and per-lane byte offsets computed
    // once, so that a load costs no vector address arithmetic.  Offsets must
    // fit 32 bits; otherwise every tile takes the form above.
    // Lane l of every load writes row q = l >> 4 of its group, position
    // l & 15, so its chunk and byte offset from the group's first row are the
    // same for all loads of all tiles.
    // (Both lane values are derived from the thread index at each use, behind
    // an opaque copy: held across the loop they would take registers the
    // kernel does not have.)
    const bool fast_ok = (long long)(63 * ks.dil + 1) * rowstride * 2 < (1ll << 31);
    const unsigned row_bytes = (unsigned)(ks.dil * rowstride * 2);
    auto load_tile_rows_fast = [&](const __bf16* base, unsigned lds_b, bool is_v, int t,
                                   int row0) {
        const unsigned slot_b = lds_b + (unsigned)((t % NSLOT) * SLOT * 2);
        unsigned tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const unsigned q = (tid >> 4) & 3;
        const unsigned chunk = (tid & 15) ^ (is_v ? 4 * q : q);
        const unsigned off = q * row_bytes + (chunk << 4);
#pragma unroll
        for (int u = 0; u < LOADS; u++) {
            const __bf16* ubase =
                base + (size_t)(ks.r + (ks.k_lo + t * BN + row0 + 4 * u) * ks.dil) * rowstride;
            SWA_DCHECK(ks.k_lo + t * BN + row0 + 4 * u + 3 <= ks.k_hi &&
                       ks.r + (ks.k_lo + t * BN + row0 + 4 * u + (int)q) * ks.dil < p.N);
            SWA_DCHECK(slot_b + (row0 / 4 + u) * GRP * 2 + 1024 <= lds_b + NSLOT * SLOT * 2);
            load_lds_x4(ubase, off, slot_b + (unsigned)((row0 / 4 + u) * GRP * 2));
        }
    };
    const int n = ks.n_tiles;
    const __bf16* my_src = grp == 0 ? kbase : vbase;
    const unsigned my_lds = grp == 0 ? k_lds_b : v_lds_b;
    const int my_row0 = (wave & 3) * 16;
    // ---- prologue: K and V of tiles 0 and 1 (group A K, group B V) -----------
    const bool my_v = grp == 1;
    if (n > 0) load_tile_rows(my_src, my_lds, my_v, 0, my_row0);
    if (n > 1) load_tile_rows(my_src, my_lds, my_v, 1, my_row0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // the query fragments have landed before the loop: an empty use makes the
    // compiler wait for them here, once, instead of at the first score MFMA
    // of every step
#pragma unroll
    for (int kc = 0; kc < KC; kc++) asm volatile("" ::"v"(qreg[kc]));
    if (grp == 1) __syncthreads();   // group B starts one phase later

    const int key_l = half * 4 + ((lane & 15) >> 2);
    const int col_l = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    f32x16 s[2];
    bf16x8 pb[4];
    bool act_prev = false;

    // V^T fragments of 16-key step tt of tile tv: rows tt*16 + key_l (+8),
    // i.e. group 4 tt + half (+2), row q = key_l & 3 of it; columns
    // db*32 + col_l .. +3, in chunk 4 db + (col_l >> 3), stored at position
    // 4 (db ^ q) + (col_l >> 3).  Per lane one base per db; tt and the +8
    // rows are immediate offsets.
    const int vq = key_l & 3;
    int vbase_db[DB];
#pragma unroll
    for (int db = 0; db < DB; db++)
        vbase_db[db] = half * GRP + vq * ROW + 32 * (db ^ vq) + 8 * (col_l >> 3) + (col_l & 7);
    auto read_v = [&](bf16x8 (&va)[DB], int tv, int tt) {
        const unsigned short* Vs = v_lds + (tv % NSLOT) * SLOT;
#pragma unroll
        for (int db = 0; db < DB; db++) {
            const i16x4 lo = lds_read_tr16(Vs + vbase_db[db] + 4 * tt * GRP);
            const i16x4 hi = lds_read_tr16(Vs + vbase_db[db] + (4 * tt + 2) * GRP);
            va[db] = __builtin_bit_cast(bf16x8,
                                        __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    // K fragments of k-steps 2g and 2g + 1 of tile tk, as [kc][kb]: row
    // kb*32 + l32 (group 8 kb + l32 / 4, row q = l32 & 3), chunk 2 kc + half
    // at position (2 kc + half) ^ q = 2 (kc ^ (q >> 1)) + (half ^ (q & 1)):
    // for even kc = 2m at 32 m + 16 (q >> 1), for odd kc at 32 m + 16 - 16 (q >> 1)
    // elements (plus 8 (half ^ (q & 1))).
    const int kq = l32 & 3;
    const int krow = (l32 >> 2) * GRP + kq * ROW + 8 * (half ^ (kq & 1));
    const int kbase_e = krow + 16 * (kq >> 1);
    const int kbase_o = krow + 16 - 16 * (kq >> 1);
    auto read_k = [&](bf16x8 (&ka)[4], int tk, int g) {
        const unsigned short* Ks = k_lds + (tk % NSLOT) * SLOT;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int kc = 2 * g + i / 2, kb = i % 2;
            const int base = (kc & 1) ? kbase_o : kbase_e;
            ka[i] = *(const bf16x8*)(Ks + base + 32 * (kc >> 1) + kb * 8 * GRP);
        }
    };
    // MFMA helpers: P V step tt of the previous tile, and k-steps 2g, 2g + 1 of
    // S^T = K Q^T
    auto pv_mfma = [&](const bf16x8 (&va)[DB], int tt) {
#pragma unroll
        for (int db = 0; db < DB; db++)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pb[tt], oacc[db], 0, 0, 0);
    };
    auto s_mfma = [&](const bf16x8 (&ka)[4], int g) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int kc = 2 * g + i / 2, kb = i % 2;
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qreg[kc], s[kb], 0, 0, 0);
        }
    };
    // The row sum is kept as four partial sums (one per 16-key step): one
    // running sum would be a chain of sixteen dependent dot products per tile,
    // and in the vector phase no other wave's work on this SIMD hides that
    // latency.
    float l_part[4] = {0.f, 0.f, 0.f, 0.f};
    // V^T fragments of the first key step of the tile whose P V comes next,
    // read at the end of the vector phase (once the scores are dead), so that
    // the matrix phase starts with its first operands in registers
    bf16x8 v0[DB];

    for (int t = 0;; t++) {
        // ======== matrix phase ==================================================
        // (debug build: this barrier and the one opening the vector phase make
        // the two groups' phases run one after the other, in an order that
        // keeps every ordering the release schedule relies on; both groups
        // pass the same number of them)
        SWA_DEBUG_BARRIER();
        __builtin_amdgcn_s_setprio(1);
        // classify tile t for this wave (wave-uniform; nothing at t = n)
        const int kt0 = ks.k_lo + t * BN;
        const int kt1 = kt0 + BN - 1;
        const bool act = t < n && !(w_first > w_last || kt0 > w_last + p.wr ||
                                    kt1 < w_first - p.wl);
        const bool need_mask =
            !(kt0 >= w_last - p.wl && kt1 <= w_first + p.wr && kt1 <= ks.k_hi);
        // P V of tile t - 1, then S of tile t.  The LDS reads run two groups of
        // four MFMAs ahead of their use, so their latency overlaps the matrix
        // work; tile t's first two K groups are read during P V.  (P V has one
        // site in the loop: a second copy for the last step makes the compiler
        // keep two copies of the accumulators.)
        bf16x8 k0[4], k1[4];
        if (act_prev) {
            bf16x8 v1[DB], v2[DB], v3[DB];
            read_v(v1, t - 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
            read_v(v2, t - 1, 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
            pv_mfma(v0, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, DB, 0);
            read_v(v3, t - 1, 3);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
            pv_mfma(v1, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, DB, 0);
            // (read also when the wave skips tile t: a harmless read of the
            // slot that keeps this block free of branches)
            read_k(k0, t, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            pv_mfma(v2, 2);
            __builtin_amdgcn_sched_group_barrier(0x008, DB, 0);
            read_k(k1, t, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            pv_mfma(v3, 3);
            __builtin_amdgcn_sched_group_barrier(0x008, DB, 0);
        }
        if (t == n) break;
        if (act) {
            if (!act_prev) {
                read_k(k0, t, 0);
                read_k(k1, t, 1);
            }
            s[0] = f32x16{};
            s[1] = f32x16{};
            bf16x8 k2[4], k3[4];
            read_k(k2, t, 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            s_mfma(k0, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            read_k(k3, t, 3);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            s_mfma(k1, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            s_mfma(k2, 2);
            s_mfma(k3, 3);
        }
        __syncthreads();

        // ======== vector phase ==================================================
        SWA_DEBUG_BARRIER();
        __builtin_amdgcn_s_setprio(0);
        // this group's rows of tile t + 2, into the slot of tile t - 1
        const bool load2 = t + 2 < n;
        if (load2) {
            if (fast_ok && ks.k_lo + (t + 3) * BN - 1 <= ks.k_hi)
                load_tile_rows_fast(my_src, my_lds, my_v, t + 2, my_row0);
            else
                load_tile_rows(my_src, my_lds, my_v, t + 2, my_row0);
#ifdef SWA_DEBUG
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // loads complete at once
#endif
        }
        if (act) {
            if (need_mask) {
                // x = key - query + wl must lie in [0, wl + wr] and the key must
                // not pass k_hi: the valid key offsets of this lane form one
                // interval [lo, hi] (an empty one moved past the tile)
                const int base = kt0 + half * 4 - qres + p.wl;
                int lo = -base;
                int hi = min(p.wl + p.wr - base, ks.k_hi - kt0 - half * 4);
                if (hi < lo) lo = hi = 1 << 20;
                const unsigned span = (unsigned)(hi - lo);
#pragma unroll
                for (int kb = 0; kb < 2; kb++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int ko = kb * 32 + (e >> 2) * 8 + (e & 3);
                        if ((unsigned)(ko - lo) > span) s[kb][e] = -INFINITY;
                    }
            }
            // running max over the lane's 32 scores: a tree of three-input
            // maxima, 15 instructions of depth 4.  (fmaxf on MFMA results
            // first quiets each operand, one more instruction per score; for
            // scores that are not NaN v_max3_f32 gives the same maximum.)
            auto max3 = [](float a, float b, float c3) {
                float r;
                asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c3));
                return r;
            };
            float m11[11];
#pragma unroll
            for (int i = 0; i < 10; i++) {
                const int e = 3 * i;
                m11[i] = max3(s[e >> 4][e & 15], s[(e + 1) >> 4][(e + 1) & 15],
                              s[(e + 2) >> 4][(e + 2) & 15]);
            }
            m11[10] = max3(s[1][14], s[1][15], s[1][15]);
            const float m4a = max3(m11[0], m11[1], m11[2]);
            const float m4b = max3(m11[3], m11[4], m11[5]);
            const float m4c = max3(m11[6], m11[7], m11[8]);
            const float m4d = max3(m11[9], m11[10], m11[10]);
            const float mlane = max3(max3(m4a, m4b, m4c), m4d, m4d);
            // the max is exchanged with lane ^ 32 only when some lane's own keys
            // pass the running max by more than the lazy bound (otherwise every
            // row keeps its max, as the exchanged max would have decided too)
            if (__any(mlane * c > m_run + kLazyRescale)) {
                const float mx = wave_max_xor32(mlane) * c;
                const float m_new = mx > m_run + kLazyRescale ? mx : m_run;
                const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
                for (int tt = 0; tt < 4; tt++) l_part[tt] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; db++) oacc[db] *= alpha;
                m_run = m_new;
            }
            const float m_use = m_run;
#pragma unroll
            for (int tt = 0; tt < 4; tt++) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    pb[tt][e] = (__bf16)fast_exp2(
                        __builtin_fmaf(s[tt >> 1][(tt & 1) * 8 + e], c, -m_use));
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const bf16x2 pr = {pb[tt][2 * e], pb[tt][2 * e + 1]};
                    l_part[tt] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_part[tt], false);
                }
            }
            read_v(v0, t, 0);
        }
        // this wave's rows of tile t + 1 (loaded a step ago) are in LDS before
        // the barrier after which they are first read; those of tile t + 2 may
        // still be in flight (vmcnt counts this wave's loads, which complete
        // in order)
        if (load2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        act_prev = act;
        __syncthreads();
    }
    __builtin_amdgcn_s_setprio(0);
    if (grp == 0) __syncthreads();   // matches group B's extra first barrier

    // ---- epilogue ---------------------------------------------------------------
    const float l_lane = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
    const float l_tot = l_lane + lane_xor32(l_lane);
    if (qpos < 0) return;
    SWA_DCHECK(qpos < p.N && hq < p.Hq);
    const float inv = 1.0f / l_tot;
    __bf16* op = (__bf16*)p.out + (((size_t)b * p.N + qpos) * p.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int jq = 0; jq < 4; jq++) {
            bf16x4 o4;
#pragma unroll
            for (int e = 0; e < 4; e++) o4[e] = (__bf16)(oacc[db][jq * 4 + e] * inv);
            *(bf16x4*)(op + db * 32 + jq * 8 + half * 4) = o4;
        }
    if (p.lse != nullptr && half == 0)
        p.lse[((size_t)b * p.Hq + hq) * p.N + qpos] =
            (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

}  // namespace

bool fwd_pp_applies(const FwdParams& p, int D_) {
    return D_ == 128 && p.hpw == 4 && p.n_global == 0 && p.kring == nullptr;
}

hipError_t launch_fwd_pp(const FwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL(swa_fwd_pp_kernel, dim3(p.n_blocks), dim3(512), 0, s, p);
    return hipGetLastError();
}

#ifdef SWA_DEBUG
SWA_DEBUG_COUNTER_READER(debug_counter_fwd_pp)
#endif

}  // namespace swa
