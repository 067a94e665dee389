// fwd_common.h -- work decomposition shared by the forward kernels.
//
// Band work items: (b, kv head, head group, residue class r, position tile).
// Positions of residue class r are i = r + m*d; a tile is bmq consecutive m.
// Its key range in residue coordinates is [max(0, m0 - wl), min(Nr-1, m1 + wr)].
// With a ring (chunked prefill, d = 1, causal) the range starts at
// max(-cache_len, m0 - wl): coordinate -1 - a is the ring entry of age a.
// Global-row work items: (b, kv head, head group, row group, key chunk).
#pragma once

#include "swa_kernels.h"

namespace swa {

struct KeyStream {
    int r, dil, Nr;      // residue class of the band (GROWS: r = 0, dil = 1, Nr = N)
    int k_lo, k_hi;      // key range (residue coordinates), inclusive
    int n_band_tiles;    // tiles of `tile_keys` keys covering [k_lo, k_hi]
    int n_tiles;         // band tiles plus gathered global-key tiles
    int n_global;
    int rhead;           // ring: next slot to write (the slot of coordinate 0)
};

struct WorkItem {
    int b, kvh, hg;
    int row0;            // first query row of the workgroup: residue coordinate
                         // (band) or index into the global list (GROWS)
    int chunk;           // GROWS only
    KeyStream ks;
};

// Band item for logical index L.  Tiles of one slab run from the last position
// tile to the first, so full-window tiles start before the short ramps.
__device__ __forceinline__ WorkItem decode_band_item(const FwdParams& p, int L, int tile_keys) {
    WorkItem w;
    int t = L % p.tiles_per_slab;
    int slab = L / p.tiles_per_slab;
    w.hg = slab % p.head_groups;
    slab /= p.head_groups;
    w.kvh = slab % p.Hkv;
    w.b = slab / p.Hkv;
    w.chunk = 0;
    t = p.tiles_per_slab - 1 - t;
    int mt;
    const int long_total = p.rem * p.tiles_long;
    if (t < long_total) {
        w.ks.r = t / p.tiles_long;
        mt = t % p.tiles_long;
        w.ks.Nr = p.qd + 1;
    } else {
        const int t2 = t - long_total;
        w.ks.r = p.rem + t2 / p.tiles_short;
        mt = t2 % p.tiles_short;
        w.ks.Nr = p.qd;
    }
    w.ks.dil = p.dil;
    const int m0 = mt * p.bmq;
    const int m_last = min(m0 + p.bmq - 1, w.ks.Nr - 1);
    w.ks.k_lo = max(0, m0 - p.wl);
    w.ks.rhead = 0;
    if (p.kring != nullptr) {
        // ring state is device data: clamp it so that no slot index can leave the ring
        const int len = min(max(p.cache_len[w.b], 0), p.W);
        w.ks.rhead = min(max(p.ring_head[w.b], 0), p.W - 1);
        w.ks.k_lo = max(-len, m0 - p.wl);
    }
    w.ks.k_hi = min(w.ks.Nr - 1, m_last + p.wr);
    w.ks.n_band_tiles = (w.ks.k_hi - w.ks.k_lo + tile_keys) / tile_keys;
    w.ks.n_global = p.n_global;
    w.ks.n_tiles = w.ks.n_band_tiles + (p.n_global + tile_keys - 1) / tile_keys;
    w.row0 = m0;
    return w;
}

// Global-row item for launch index L; rows_wg global rows per workgroup.
__device__ __forceinline__ WorkItem decode_grows_item(const FwdParams& p, int L, int rows_wg,
                                                      int tile_keys) {
    WorkItem w;
    w.chunk = L % p.g_nchunks;
    L /= p.g_nchunks;
    const int rg = L % p.g_rowgroups;
    L /= p.g_rowgroups;
    w.hg = L % p.head_groups;
    L /= p.head_groups;
    w.kvh = L % p.Hkv;
    w.b = L / p.Hkv;
    const int g_first = rg * rows_wg;
    const int g_last = min(g_first + rows_wg, p.n_global) - 1;
    w.ks.r = 0;
    w.ks.dil = 1;
    w.ks.Nr = p.N;
    w.ks.k_lo = w.chunk * p.g_chunk;
    w.ks.k_hi = min(p.N, (w.chunk + 1) * p.g_chunk) - 1;
    if (p.causal) w.ks.k_hi = min(w.ks.k_hi, p.gpos[g_last]);  // gpos is sorted
    w.ks.n_band_tiles =
        w.ks.k_hi >= w.ks.k_lo ? (w.ks.k_hi - w.ks.k_lo + tile_keys) / tile_keys : 0;
    w.ks.n_tiles = w.ks.n_band_tiles;
    w.ks.n_global = p.n_global;
    w.ks.rhead = 0;
    w.row0 = g_first;
    return w;
}

// Ring slot of a negative residue coordinate kk (>= -W): the entry of age
// -1 - kk, written ring_head - 1 - age (mod W).
__device__ __forceinline__ int ring_slot(const KeyStream& ks, int kk, int W) {
    const int s = ks.rhead + kk;
    return s < 0 ? s + W : s;
}

// Absolute position of key `key` of tile `j`, or -1 when the slot is padding.
__device__ __forceinline__ int key_position(const KeyStream& ks, const FwdParams& p, int j,
                                            int key, int tile_keys, bool grows) {
    if (grows || j < ks.n_band_tiles) {
        const int kk = ks.k_lo + j * tile_keys + key;
        return kk <= ks.k_hi ? ks.r + kk * ks.dil : -1;
    }
    const int gi = (j - ks.n_band_tiles) * tile_keys + key;
    return gi < ks.n_global ? p.gpos[gi] : -1;
}

// Does key (absolute position g) of a gathered global tile count for a query
// at residue coordinate mq of class r?  Not if the band already holds it, nor
// (causal) if it lies in the query's future.
__device__ __forceinline__ bool global_key_visible(const FwdParams& p, const KeyStream& ks,
                                                   int g, int mq, int qpos) {
    bool inband = false;
    if (g % ks.dil == ks.r) {
        const int dl = g / ks.dil - mq;
        inband = dl >= -p.wl && dl <= p.wr;
    }
    return !inband && (!p.causal || g <= qpos);
}

}  // namespace swa
