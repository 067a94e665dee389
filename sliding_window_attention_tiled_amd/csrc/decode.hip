// decode.hip -- ring-buffer KV append, split-K decode and the partial combine.
//
// The ring (intelliparadigm.com, section 3.1 "cache mechanism": write at
// idx % size, then advance; aiqz.cc, "inference optimisation": only the last W
// keys/values are kept) holds W slots per (sequence, kv head), contiguous in
// memory, so one decode step streams each (b, kv head) slab once.  Decode is
// bound by that stream (about 4 flop per byte): the slab is split into
// `splits` slot ranges, one workgroup each, and every wave of a workgroup
// walks its own 32-slot chunks.  The G query heads of the kv head form the
// columns of a 16-column MFMA tile, so the K and V of each slot are read once
// for all heads.  Slots are visited in physical order (keys carry no position,
// so order does not matter); a slot counts when its age
// (ring_head - 1 - slot) mod W is below cache_len.  Each workgroup writes one
// partial (acc, m, l) per head and the combine kernel merges the splits; with
// a single split the workgroup holds the whole row and writes out and lse
// itself.  Sink entries are walked by the first split of each (b, kv head).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "swa_kernels.h"

namespace swa {
namespace {

// ---- ring append ---------------------------------------------------------------
// One workgroup per sequence: copy k_new/v_new into slot ring_head[b], then
// advance ring_head and cache_len once every lane has read the old head.
__global__ __launch_bounds__(256) void kv_append_kernel(unsigned char* kc, unsigned char* vc,
                                                        const unsigned char* kn,
                                                        const unsigned char* vn,
                                                        int32_t* head, int32_t* len, int Hkv,
                                                        int W, int row_bytes) {
    const int b = blockIdx.x;
    SWA_DCHECK(head[b] >= 0 && head[b] < W && len[b] >= 0 && len[b] <= W);
    const int slot = min(max(head[b], 0), W - 1);  // device data: keep the write in the ring
    const int chunks = Hkv * row_bytes / 16;  // 16-byte chunks per tensor
    for (int ci = threadIdx.x; ci < chunks; ci += blockDim.x) {
        const int h = ci / (row_bytes / 16), c = ci % (row_bytes / 16);
        const size_t src = ((size_t)b * Hkv + h) * row_bytes + c * 16;
        const size_t dst = (((size_t)b * Hkv + h) * W + slot) * row_bytes + c * 16;
        *(u32x4*)(kc + dst) = *(const u32x4*)(kn + src);
        *(u32x4*)(vc + dst) = *(const u32x4*)(vn + src);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        head[b] = slot + 1 == W ? 0 : slot + 1;
        len[b] = min(max(len[b], 0) + 1, W);
    }
}

// Chunk append: the last m = min(n, W) tokens of k, v [B][n][Hkv][row] go to
// slots (ring_head + t) mod W (t = n - m .. n - 1), which is what n single
// appends leave behind.  One thread per 16-byte piece, `bps` workgroups per
// sequence; the state update runs as a second kernel so that every copy has
// read the old ring_head.
__global__ __launch_bounds__(256) void kv_append_chunk_kernel(
    unsigned char* kc, unsigned char* vc, const unsigned char* k, const unsigned char* v,
    const int32_t* head, int Hkv, int W, int n, int m, int row_bytes, int bps) {
    const int b = blockIdx.x / bps;
    const int cpr = row_bytes / 16;               // 16-byte chunks per row
    const int64_t total = (int64_t)m * Hkv * cpr;  // chunks of this sequence
    const int64_t ci = (int64_t)(blockIdx.x % bps) * blockDim.x + threadIdx.x;
    if (ci >= total) return;
    const int c = (int)(ci % cpr);
    const int h = (int)((ci / cpr) % Hkv);
    const int64_t t = n - m + ci / ((int64_t)cpr * Hkv);
    SWA_DCHECK(head[b] >= 0 && head[b] < W);
    const int64_t h0 = min(max(head[b], 0), W - 1);
    const int64_t slot = (h0 + t) % W;
    const size_t src = (((size_t)b * n + t) * Hkv + h) * row_bytes + c * 16;
    const size_t dst = (((size_t)b * Hkv + h) * W + slot) * row_bytes + c * 16;
    *(u32x4*)(kc + dst) = *(const u32x4*)(k + src);
    *(u32x4*)(vc + dst) = *(const u32x4*)(v + src);
}

__global__ __launch_bounds__(64) void ring_advance_kernel(int32_t* head, int32_t* len, int B,
                                                         int W, int n) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    SWA_DCHECK(head[b] >= 0 && head[b] < W);
    const int64_t h0 = min(max(head[b], 0), W - 1);
    head[b] = (int32_t)((h0 + n) % W);
    len[b] = (int32_t)min<int64_t>((int64_t)max(len[b], 0) + n, W);
}

// ---- paged cache append ----------------------------------------------------------
// Positions seq_len[b] + t (t = n - m .. n - 1, m = min(n, W)) of sequence b go
// to their page block_table[b][(pos / P) % nb], slot pos % P.  Page ids are
// device data: they are clamped into the pool so that no write leaves it.
__global__ __launch_bounds__(256) void kv_append_paged_kernel(
    unsigned char* kpool, unsigned char* vpool, const unsigned char* k, const unsigned char* v,
    const int32_t* table, const int32_t* seq_len, int Hkv, int n_pages, int page_shift, int nb,
    int n, int m, int row_bytes, int bps) {
    const int b = blockIdx.x / bps;
    const int cpr = row_bytes / 16;
    const int64_t total = (int64_t)m * Hkv * cpr;
    const int64_t ci = (int64_t)(blockIdx.x % bps) * blockDim.x + threadIdx.x;
    if (ci >= total) return;
    const int c = (int)(ci % cpr);
    const int h = (int)((ci / cpr) % Hkv);
    const int64_t t = n - m + ci / ((int64_t)cpr * Hkv);
    const int64_t pos = (int64_t)max(seq_len[b], 0) + t;
    int page = table[(size_t)b * nb + (int)((pos >> page_shift) % nb)];
    SWA_DCHECK(seq_len[b] >= 0 && page >= 0 && page < n_pages);
    page = min(max(page, 0), n_pages - 1);
    const int64_t slot = pos & ((1 << page_shift) - 1);
    const size_t src = (((size_t)b * n + t) * Hkv + h) * row_bytes + c * 16;
    const size_t dst = ((((size_t)page * Hkv + h) << page_shift) + slot) * row_bytes + c * 16;
    *(u32x4*)(kpool + dst) = *(const u32x4*)(k + src);
    *(u32x4*)(vpool + dst) = *(const u32x4*)(v + src);
}

__global__ __launch_bounds__(64) void seq_advance_kernel(int32_t* seq_len, int B, int n) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) seq_len[b] = max(seq_len[b], 0) + n;
}

// Element offset of the row of window index i (0 = oldest live position) in
// the page pool, for (b, kv head) of a paged decode.
__device__ __forceinline__ size_t paged_row(const DecodeParams& p, int b, int kvh, int pos0,
                                            int i, int D) {
    const int pos = pos0 + i;
    int page = p.block_table[(size_t)b * p.nb + ((pos >> p.page_shift) % p.nb)];
    SWA_DCHECK(page >= 0 && page < p.n_pages);
    page = min(max(page, 0), p.n_pages - 1);
    return ((((size_t)page * p.Hkv + kvh) << p.page_shift) + (pos & ((1 << p.page_shift) - 1))) *
           D;
}

// ---- bf16 split decode on MFMA ----------------------------------------------------
constexpr int CH = 32;        // slots per chunk
constexpr int DNT = 256;      // 4 waves

template <int D>
struct DecCfg {
    static constexpr int PITCH = D + 8;               // bf16 per LDS row
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int PER_LANE = CH * CPR / 64;    // 16-byte chunks per lane per tensor
    static constexpr int WAVE_ELEMS = 2 * CH * PITCH; // K and V of one chunk
};

// PAGED: the W slots are the window positions seq_len - min(seq_len, W) + i,
// read through the block table; otherwise the ring's physical slots.
template <int D, bool PAGED>
__global__ __launch_bounds__(DNT, 2) void decode_bf16_kernel(const DecodeParams p) {
    using C = DecCfg<D>;
    constexpr int KS = D / 32;   // 32-deep k-steps of S^T = K Q^T (16x16x32)
    constexpr int DB = D / 16;   // 16-row blocks of O^T
    __shared__ __attribute__((aligned(16))) unsigned short smem[4 * C::WAVE_ELEMS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int grp = lane >> 4;

    // work item: (b, kv head, head block, split); splits fastest
    int L = blockIdx.x;
    const int s = L % p.splits;
    L /= p.splits;
    const int hblocks = (p.group + 15) / 16;
    const int hb = L % hblocks;
    L /= hblocks;
    const int kvh = L % p.Hkv;
    const int b = L / p.Hkv;

    const int head_col = hb * 16 + l16;          // this lane's query head within the group
    const bool head_ok = head_col < p.group;
    const int hq = kvh * p.group + head_col;

    const int W = p.W;
    const int ring_head = PAGED ? 0 : p.ring_head[b];
    // paged: live window positions pos0 .. pos0 + n_live - 1
    const int seq_n = PAGED ? max(p.seq_len[b], 0) : 0;
    const int n_live = min(seq_n, W);
    const int pos0 = seq_n - n_live;
    const int cache_len = PAGED ? n_live : p.cache_len[b];
    const bool full = cache_len >= W;
    SWA_DCHECK(PAGED || (ring_head >= 0 && ring_head < W && cache_len >= 0 && cache_len <= W));

    // ring slots of this wave
    const int s_lo = s * p.slots_per_split;
    const int s_hi = min(W, s_lo + p.slots_per_split);
    const int per_wave = (s_hi - s_lo + 3) / 4;
    const int w_lo = min(s_hi, s_lo + wave * per_wave);
    const int w_hi = min(s_hi, w_lo + per_wave);
    const int n_chunks = (w_hi - w_lo + CH - 1) / CH;
    // the first split also walks the sink entries (all valid), a quarter per
    // wave, as chunks n_chunks .. n_all - 1 of the wave
    const int n_sk = (!PAGED && s == 0) ? p.n_sink : 0;
    const int k_per = (n_sk + 3) / 4;
    const int k_lo = min(n_sk, wave * k_per);
    const int k_hi = min(n_sk, k_lo + k_per);
    const int n_all = n_chunks + (k_hi - k_lo + CH - 1) / CH;

    // Q^T as the B operand: lane holds head column l16, dims ks*32 + grp*8 .. +7
    bf16x8 qreg[KS];
    {
        const __bf16* qp = (const __bf16*)p.q + ((size_t)b * p.Hq + (head_ok ? hq : 0)) * D + grp * 8;
#pragma unroll
        for (int k = 0; k < KS; k++)
            qreg[k] = head_ok ? *(const bf16x8*)(qp + k * 32)
                              : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    const size_t bk = (size_t)b * p.Hkv + kvh;
    const __bf16* kbase = (const __bf16*)p.kcache + (PAGED ? 0 : bk * W * D);
    const __bf16* vbase = (const __bf16*)p.vcache + (PAGED ? 0 : bk * W * D);
    const __bf16* ksbase = n_sk > 0 ? (const __bf16*)p.ksink + bk * n_sk * D : kbase;
    const __bf16* vsbase = n_sk > 0 ? (const __bf16*)p.vsink + bk * n_sk * D : vbase;
    unsigned short* Ks = smem + wave * C::WAVE_ELEMS;
    unsigned short* Vs = Ks + CH * C::PITCH;

    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; db++) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kEmptyMax, l_run = 0.f;
    const float c = p.scale_log2;

    // paged: the wave's pages are looked up once, one per lane (block fb + lane),
    // and each key finds its page with a lane permute, so a chunk's loads do not
    // wait on a table read.  Wave ranges spanning more than 64 pages (pages
    // shorter than a 64th of the range) read the table per key instead.
    int fb = 0, my_page = 0;
    bool lane_pages = false;
    if (PAGED && w_lo < w_hi) {
        fb = (pos0 + w_lo) >> p.page_shift;
        const int nblk = ((pos0 + w_hi - 1) >> p.page_shift) - fb + 1;
        lane_pages = nblk <= 64;
        if (lane_pages && lane < nblk) {
            const int pg = p.block_table[(size_t)b * p.nb + ((fb + lane) % p.nb)];
            SWA_DCHECK(pg >= 0 && pg < p.n_pages);
            my_page = min(max(pg, 0), p.n_pages - 1);
        }
    }
    // page of window index i from the lane copies; every lane takes part in the
    // permute (lanes whose key is out of range discard the result)
    auto lane_page = [&](int i) -> int {
        return __builtin_amdgcn_ds_bpermute((((pos0 + i) >> p.page_shift) - fb) << 2, my_page);
    };
    auto page_row = [&](int i, int pg) -> size_t {
        const int pos = pos0 + i;
        if (!lane_pages) return paged_row(p, b, kvh, pos0, i, D);
        return ((((size_t)pg * p.Hkv + kvh) << p.page_shift) +
                (pos & ((1 << p.page_shift) - 1))) * D;
    };

    u32x4 kr[C::PER_LANE], vr[C::PER_LANE];
    // chunk ck of the wave: ring slots, or sink entries past the ring chunks
    auto chunk_base = [&](int ck) -> int {
        return !PAGED && ck >= n_chunks ? k_lo + (ck - n_chunks) * CH : w_lo + ck * CH;
    };
    auto chunk_end = [&](int ck) -> int { return !PAGED && ck >= n_chunks ? k_hi : w_hi; };
    // A ring slot that holds no entry (age >= cache_len) is not read: its
    // bytes are whatever the caller's buffer held, and a zero weight times a
    // NaN or infinity there would still reach the output.
    auto slot_live = [&](int slot) {
        int age = ring_head - 1 - slot;
        if (age < 0) age += W;
        return age < cache_len;
    };
    auto load_chunk = [&](int ck) {
        const bool sk = !PAGED && ck >= n_chunks;
        const int base = chunk_base(ck), hi = chunk_end(ck);
        const __bf16* kb = sk ? ksbase : kbase;
        const __bf16* vb = sk ? vsbase : vbase;
#pragma unroll
        for (int u = 0; u < C::PER_LANE; u++) {
            const int ci = lane + u * 64;
            const int key = ci / C::CPR, cc = ci % C::CPR;
            const int pg = PAGED && lane_pages ? lane_page(base + key) : 0;
            const bool live = PAGED ? base + key < n_live : (sk || full || slot_live(base + key));
            if (base + key < hi && live) {
                SWA_DCHECK(base + key >= 0 && base + key < (sk ? n_sk : W));
                const size_t off = (PAGED ? page_row(base + key, pg)
                                          : (size_t)(base + key) * D) + cc * 8;
                kr[u] = __builtin_nontemporal_load((const u32x4*)(kb + off));
                vr[u] = __builtin_nontemporal_load((const u32x4*)(vb + off));
            } else {
                kr[u] = u32x4{0u, 0u, 0u, 0u};
                vr[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    if (n_all > 0) load_chunk(0);
    for (int ck = 0; ck < n_all; ck++) {
        // stage the chunk in this wave's LDS area (natural [slot][d] layout)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < C::PER_LANE; u++) {
            const int ci = lane + u * 64;
            const int key = ci / C::CPR, cc = ci % C::CPR;
            *(u32x4*)(Ks + key * C::PITCH + cc * 8) = kr[u];
            *(u32x4*)(Vs + key * C::PITCH + cc * 8) = vr[u];
        }
        __builtin_amdgcn_wave_barrier();
        if (ck + 1 < n_all) load_chunk(ck + 1);

        // S^T = K Q^T: two 16-slot blocks
        f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int k = 0; k < KS; k++) {
                const bf16x8 a = *(const bf16x8*)(Ks + (kb * 16 + l16) * C::PITCH + k * 32 + grp * 8);
                sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[k], sc[kb], 0, 0, 0);
            }
        // mask slots beyond the wave range or older than cache_len
        const bool sk = !PAGED && ck >= n_chunks;
        const int base = chunk_base(ck), hi = chunk_end(ck);
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int slot = base + kb * 16 + grp * 4 + e;
                bool valid = slot < hi;
                if (PAGED) {
                    valid = valid && slot < n_live;
                } else if (!full && !sk) {
                    int age = ring_head - 1 - slot;
                    if (age < 0) age += W;
                    valid = valid && age < cache_len;
                }
                if (!valid) sc[kb][e] = -INFINITY;
            }
        // online softmax for this lane's head column (lanes l16, l16+16, +32, +48 agree)
        float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mx *= c;
        const bool up = mx > m_run + kLazyRescale;
        const float m_use = up ? mx : m_run;
        if (__any(up)) {
            const float alpha = fast_exp2(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; db++) oacc[db] *= alpha;
        }
        m_run = m_use;
        // weights rounded to bf16 (the B operand of P V); the running sum adds
        // those rounded weights, so out is normalised by exactly the weights
        // it was built from, as in the forward
        bf16x8 pb;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                pb[kb * 4 + e] = (__bf16)fast_exp2(__builtin_fmaf(sc[kb][e], c, -m_use));
        {
            const __bf16 one = (__bf16)1.0f;
            const bf16x2 ones = {one, one};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const bf16x2 pr = {pb[2 * e], pb[2 * e + 1]};
                l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
            }
        }
        // O^T += V^T P^T: slot (grp*8 + t) of the B operand is key grp*4 + t (t < 4)
        // or 16 + grp*4 + (t - 4); V^T comes from transposing LDS reads.
#pragma unroll
        for (int db = 0; db < DB; db++) {
            const int col = db * 16 + 4 * (lane & 3);
            const int key = grp * 4 + (l16 >> 2);
            const i16x4 lo = lds_read_tr16(Vs + key * C::PITCH + col);
            const i16x4 hi = lds_read_tr16(Vs + (key + 16) * C::PITCH + col);
            const bf16x8 a =
                __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, oacc[db], 0, 0, 0);
        }
    }

    // ---- merge the 4 lane groups, then the 4 waves, into one partial per head
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    __syncthreads();  // staging areas are free now
    float* red = (float*)smem;                       // [4 waves][16 heads][D]
    float* red_ml = red + 4 * 16 * D;                // [4 waves][16 heads][2]
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
        for (int e = 0; e < 4; e++)
            red[(wave * 16 + l16) * D + db * 16 + grp * 4 + e] = oacc[db][e];
    if (grp == 0) {
        red_ml[(wave * 16 + l16) * 2] = m_run;
        red_ml[(wave * 16 + l16) * 2 + 1] = l_run;
    }
    __syncthreads();
    const int heads_here = min(16, p.group - hb * 16);
    for (int idx = threadIdx.x; idx < heads_here * D; idx += DNT) {
        const int h = idx / D, d = idx % D;
        float M = kEmptyMax;
#pragma unroll
        for (int w = 0; w < 4; w++) M = fmaxf(M, red_ml[(w * 16 + h) * 2]);
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const float f = fast_exp2(red_ml[(w * 16 + h) * 2] - M);
            acc += f * red[(w * 16 + h) * D + d];
            lsum += f * red_ml[(w * 16 + h) * 2 + 1];
        }
        const int hq2 = kvh * p.group + hb * 16 + h;
        if (p.out != nullptr) {
            // one split: this is the whole row, finished as the combine would
            const size_t row = (size_t)b * p.Hq + hq2;
            const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
            ((__bf16*)p.out)[row * D + d] = (__bf16)(acc * inv);
            if (p.lse != nullptr && d == 0)
                p.lse[row] = lsum > 0.f ? (M + __builtin_amdgcn_logf(lsum)) * kLn2 : -INFINITY;
        } else {
            float* rec = p.partials + (((size_t)b * p.Hq + hq2) * p.splits + s) * (D + kPartialPad);
            rec[d] = acc;
            if (d == 0) {
                rec[D] = M;
                rec[D + 1] = lsum;
            }
        }
    }
}

// ---- float32 split decode on the vector ALUs -------------------------------------
// One wave per (b, query head, split); lanes 16*r .. 16*r+15 share a slot, each
// lane a D/16 slice of it; four slots per step.
template <int D, bool PAGED>
__global__ __launch_bounds__(64) void decode_f32_kernel(const DecodeParams p) {
    constexpr int DL = D / 16;
    const int lane = threadIdx.x;
    const int sub = lane >> 4, part = lane & 15;
    int L = blockIdx.x;
    const int s = L % p.splits;
    L /= p.splits;
    const int hq = L % p.Hq;
    const int b = L / p.Hq;
    const int kvh = hq / p.group;
    const bool sink_split = !PAGED && s >= p.ring_splits;  // sink entries: all valid
    const int W = p.W;
    const int ring_head = PAGED ? 0 : p.ring_head[b];
    const int seq_n = PAGED ? max(p.seq_len[b], 0) : 0;
    const int n_live = min(seq_n, W);
    const int pos0 = seq_n - n_live;
    const int cache_len = sink_split ? W : PAGED ? n_live : p.cache_len[b];
    const int src_slots = sink_split ? p.n_sink : W;
    const int s_lo = sink_split ? 0 : s * p.slots_per_split;
    const int s_hi = sink_split ? p.n_sink : min(W, s_lo + p.slots_per_split);

    float q[DL];
    const float* qp = (const float*)p.q + ((size_t)b * p.Hq + hq) * D + part * DL;
#pragma unroll
    for (int d = 0; d < DL; d++) q[d] = qp[d];
    const size_t slab = PAGED ? 0 : ((size_t)b * p.Hkv + kvh) * src_slots;
    const float* kbase = (const float*)(sink_split ? p.ksink : p.kcache) + slab * D + part * DL;
    const float* vbase = (const float*)(sink_split ? p.vsink : p.vcache) + slab * D + part * DL;
    float acc[DL];
#pragma unroll
    for (int d = 0; d < DL; d++) acc[d] = 0.f;
    float m_run = kEmptyMax, l_run = 0.f;
    const float c = p.scale_log2;
    for (int base = s_lo; base < s_hi; base += 4) {
        const int slot = base + sub;
        bool valid = slot < s_hi;
        if (PAGED) {
            valid = valid && slot < n_live;
        } else if (valid && cache_len < W) {
            int age = ring_head - 1 - slot;
            if (age < 0) age += W;
            valid = age < cache_len;
        }
        const size_t row = PAGED ? (valid ? paged_row(p, b, kvh, pos0, slot, D) : 0)
                                 : (size_t)slot * D;
        float dot = 0.f;
        if (PAGED ? valid : slot < s_hi) {
#pragma unroll
            for (int d = 0; d < DL; d++) dot = __builtin_fmaf(q[d], kbase[row + d], dot);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) dot += __shfl_xor(dot, o);
        const float sv = valid ? dot * c : -INFINITY;
        const bool up = sv > m_run + kLazyRescale;
        const float m_use = up ? sv : m_run;
        if (up) {
            const float alpha = fast_exp2(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < DL; d++) acc[d] *= alpha;
        }
        m_run = m_use;
        const float pk = fast_exp2(sv - m_use);
        l_run += pk;
        if (valid) {
#pragma unroll
            for (int d = 0; d < DL; d++) acc[d] = __builtin_fmaf(pk, vbase[row + d], acc[d]);
        }
    }
    // merge the four slot lanes (sub = 0..3) of each dim slice
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
        const float m_o = __shfl_xor(m_run, o);
        const float l_o = __shfl_xor(l_run, o);
        const float M = fmaxf(m_run, m_o);
        const float fa = fast_exp2(m_run - M), fb = fast_exp2(m_o - M);
#pragma unroll
        for (int d = 0; d < DL; d++) {
            const float a_o = __shfl_xor(acc[d], o);
            acc[d] = acc[d] * fa + a_o * fb;
        }
        l_run = l_run * fa + l_o * fb;
        m_run = M;
    }
    if (sub == 0) {
        float* rec = p.partials + (((size_t)b * p.Hq + hq) * p.splits + s) * (D + kPartialPad);
#pragma unroll
        for (int d = 0; d < DL; d++) rec[part * DL + d] = acc[d];
        if (part == 0) {
            rec[D] = m_run;
            rec[D + 1] = l_run;
        }
    }
}

// ---- merge split partials ------------------------------------------------------------
// One wave per output row: M = max m_s, L = sum l_s 2^(m_s - M),
// out = sum acc_s 2^(m_s - M) / L, lse = (M + log2 L) ln 2.  A row with no keys
// (L == 0) gets out = 0 and lse = -inf.  The (m, l) pairs are read one split
// per lane and reduced across the wave; the acc records are read with eight
// splits' loads in flight, each lane holding D / 64 dimensions.
template <int D, typename OutT>
__global__ __launch_bounds__(64) void combine_kernel(const CombineParams p) {
    constexpr int RP = D + kPartialPad;  // floats per record
    constexpr int U = 8;                 // splits per batch of loads
    const int row = blockIdx.x;
    const int lane = threadIdx.x;
    const float* rec0 = p.partials + (size_t)row * p.splits * RP;
    float M = kEmptyMax;
    for (int s = lane; s < p.splits; s += 64) M = fmaxf(M, rec0[(size_t)s * RP + D]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f;
    float acc[D / 64];
#pragma unroll
    for (int i = 0; i < D / 64; i++) acc[i] = 0.f;
    for (int s0 = 0; s0 < p.splits; s0 += 64) {
        // weight of split s0 + lane, then its share of L
        const int s = s0 + lane;
        float f = 0.f;
        if (s < p.splits) {
            const float* rec = rec0 + (size_t)s * RP;
            f = fast_exp2(rec[D] - M);
            L += f * rec[D + 1];
        }
        const int n = min(64, p.splits - s0);
        const float* base = rec0 + (size_t)s0 * RP + lane;
        int t = 0;
        for (; t + U <= n; t += U) {
            float v[U][D / 64];
#pragma unroll
            for (int u = 0; u < U; u++)
#pragma unroll
                for (int i = 0; i < D / 64; i++) v[u][i] = base[(size_t)(t + u) * RP + i * 64];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const float fu = __shfl(f, t + u);
#pragma unroll
                for (int i = 0; i < D / 64; i++) acc[i] += fu * v[u][i];
            }
        }
        for (; t < n; t++) {
            const float fu = __shfl(f, t);
#pragma unroll
            for (int i = 0; i < D / 64; i++) acc[i] += fu * base[(size_t)t * RP + i * 64];
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    size_t out_off, lse_off;
    if (p.mode == 0) {
        out_off = (size_t)row * D;
        lse_off = row;
    } else {
        const int gi = row % p.n_global;
        const int bh = row / p.n_global;  // b * Hq + h
        const int b = bh / p.Hq, h = bh % p.Hq;
        const int pos = p.gpos[gi];
        out_off = (((size_t)b * p.N + pos) * p.Hq + h) * D;
        lse_off = (size_t)bh * p.N + pos;
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    OutT* op = (OutT*)p.out + out_off;
#pragma unroll
    for (int i = 0; i < D / 64; i++) op[lane + i * 64] = (OutT)(acc[i] * inv);
    if (p.lse != nullptr && lane == 0)
        p.lse[lse_off] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_kv_append(void* kc, void* vc, const void* kn, const void* vn, int32_t* head,
                            int32_t* len, int B, int Hkv, int W, int D, int elem_bytes,
                            hipStream_t s) {
    hipLaunchKernelGGL(kv_append_kernel, dim3(B), dim3(256), 0, s, (unsigned char*)kc,
                       (unsigned char*)vc, (const unsigned char*)kn, (const unsigned char*)vn,
                       head, len, Hkv, W, D * elem_bytes);
    return hipGetLastError();
}

hipError_t launch_kv_append_chunk(void* kc, void* vc, const void* k, const void* v,
                                  int32_t* head, int32_t* len, int B, int Hkv, int W, int n,
                                  int D, int elem_bytes, hipStream_t s) {
    const int m = n < W ? n : W;
    const int row_bytes = D * elem_bytes;
    const int64_t chunks = (int64_t)m * Hkv * (row_bytes / 16);
    const int64_t bps = (chunks + 255) / 256;  // workgroups per sequence
    if (bps * B > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_append_chunk_kernel, dim3((unsigned)(bps * B)), dim3(256), 0, s,
                       (unsigned char*)kc, (unsigned char*)vc, (const unsigned char*)k,
                       (const unsigned char*)v, (const int32_t*)head, Hkv, W, n, m, row_bytes,
                       (int)bps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ring_advance_kernel, dim3((B + 63) / 64), dim3(64), 0, s, head, len, B, W,
                       n);
    return hipGetLastError();
}

hipError_t launch_kv_append_paged(void* kpool, void* vpool, const void* k, const void* v,
                                  const int32_t* block_table, int32_t* seq_len, int B, int Hkv,
                                  int n_pages, int page_shift, int nb, int W, int n, int D,
                                  int elem_bytes, hipStream_t s) {
    const int m = n < W ? n : W;
    const int row_bytes = D * elem_bytes;
    const int64_t bps = ((int64_t)m * Hkv * (row_bytes / 16) + 255) / 256;
    if (bps * B > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_append_paged_kernel, dim3((unsigned)(bps * B)), dim3(256), 0, s,
                       (unsigned char*)kpool, (unsigned char*)vpool, (const unsigned char*)k,
                       (const unsigned char*)v, block_table, (const int32_t*)seq_len, Hkv,
                       n_pages, page_shift, nb, n, m, row_bytes, (int)bps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(seq_advance_kernel, dim3((B + 63) / 64), dim3(64), 0, s, seq_len, B, n);
    return hipGetLastError();
}

template <bool PAGED>
void launch_decode_bf16_t(const DecodeParams& p, int D, hipStream_t s) {
    const int grid = p.B * p.Hkv * ((p.group + 15) / 16) * p.splits;
    if (D == 128)
        hipLaunchKernelGGL((decode_bf16_kernel<128, PAGED>), dim3(grid), dim3(DNT), 0, s, p);
    else
        hipLaunchKernelGGL((decode_bf16_kernel<64, PAGED>), dim3(grid), dim3(DNT), 0, s, p);
}

template <bool PAGED>
void launch_decode_f32_t(const DecodeParams& p, int D, hipStream_t s) {
    const int grid = p.B * p.Hq * p.splits;
    if (D == 128)
        hipLaunchKernelGGL((decode_f32_kernel<128, PAGED>), dim3(grid), dim3(64), 0, s, p);
    else
        hipLaunchKernelGGL((decode_f32_kernel<64, PAGED>), dim3(grid), dim3(64), 0, s, p);
}

hipError_t launch_decode_bf16(const DecodeParams& p, int D, bool paged, hipStream_t s) {
    if (paged) launch_decode_bf16_t<true>(p, D, s);
    else launch_decode_bf16_t<false>(p, D, s);
    return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeParams& p, int D, bool paged, hipStream_t s) {
    if (paged) launch_decode_f32_t<true>(p, D, s);
    else launch_decode_f32_t<false>(p, D, s);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int D, int dtype, hipStream_t s) {
    if (p.rows == 0) return hipSuccess;
    if (dtype == SWA_BF16) {
        if (D == 128)
            hipLaunchKernelGGL((combine_kernel<128, __bf16>), dim3(p.rows), dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL((combine_kernel<64, __bf16>), dim3(p.rows), dim3(64), 0, s, p);
    } else {
        if (D == 128)
            hipLaunchKernelGGL((combine_kernel<128, float>), dim3(p.rows), dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL((combine_kernel<64, float>), dim3(p.rows), dim3(64), 0, s, p);
    }
    return hipGetLastError();
}

#ifdef SWA_DEBUG
SWA_DEBUG_COUNTER_READER(debug_counter_decode)
#endif

}  // namespace swa
