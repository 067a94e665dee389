// swa_kernels.h -- parameter blocks shared by the host API (swa_api.cpp) and
// the HIP kernels of libswa.so.  Internal to the library.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/swa.h"

namespace swa {

// Partial softmax state written by split-K passes and merged by the combine
// kernel: acc[D] (unnormalised weighted sum of v), m (running max of the
// scaled scores, base-2 units), l (sum of 2^(s - m)).  Records are padded to
// a multiple of 16 bytes.
constexpr int kPartialPad = 4;
inline int partial_floats(int D) { return D + kPartialPad; }

// Upper bound of score contributions kept without rescaling: the running max
// is only moved when a tile's max exceeds it by more than this (base-2 units),
// so unnormalised weights stay <= 2^kLazyRescale.
constexpr float kLazyRescale = 8.0f;

// One forward launch.  Positions are split into residue classes r = i mod d;
// inside a class the dilated window is an ordinary window over m = (i - r) / d.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;        // may be null
    float* partials;   // global-row partials [B][Hq][n_global][g_nchunks][D+4]
    int B, Hq, Hkv, N, group;   // group = Hq / Hkv
    int wl, wr, dil, causal;
    float scale_log2;  // scale * log2(e)
    // residue classes: N = qd * dil + rem; classes r < rem hold qd + 1 positions
    int qd, rem;
    // band work decomposition
    int hpw;           // query heads per workgroup (1, 2 or 4)
    int bmq;           // query positions per workgroup (per residue class)
    int tiles_long, tiles_short;  // position tiles in a long / short residue class
    int tiles_per_slab;           // all tiles of one (b, kv head, head group)
    int head_groups;              // group / hpw
    int n_blocks;                 // grid size of the band launch
    int rotate;                   // bf16 band launch: walk band tiles rotated (set at launch)
    // global tokens (sorted, unique)
    int n_global;
    int g_chunk;       // keys per split of a global row
    int g_nchunks;     // splits per global row
    int g_rowgroups;   // workgroups needed to cover n_global rows
    int32_t gpos[SWA_MAX_GLOBAL];
    // chunked prefill: keys before the chunk come from a ring [B][Hkv][W][D]
    // (null kring: none).  Residue coordinates -1, -2, ... are ring ages 0, 1, ...
    const void* kring;
    const void* vring;
    const int32_t* ring_head;
    const int32_t* cache_len;
    int W;
};

// One backward launch: the forward's band plan (no global tokens) in f, plus
// the upstream gradient, the forward's lse, the per-row dot(dout, out) and
// the gradient outputs.  The key-major pass tiles each residue class's keys
// in blocks of bmk and visits the query positions whose windows reach them.
struct BwdParams {
    FwdParams f;
    const void* out;
    const void* dout;
    float* delta;      // [B][Hq][N]: sum_d dout * out per query row
    void* dq;
    void* dk;
    void* dv;
    float scale;       // multiplier of q.k (dq, dk carry it)
    int bmk;                        // keys per key-major workgroup
    int ktiles_long, ktiles_short;  // key blocks in a long / short residue class
    int ktiles_per_slab;            // key blocks of one (b, kv head)
    int k_blocks;                   // grid of the key-major pass
};

// The backward's pairs outside the band that global tokens add (global rows
// with every key, every row with the global keys); see bwd_global.hip.
// Global rows (keys) per workgroup of the passes whose items are global tokens.
constexpr int kGlobalBwdItems = 16;
struct GlobalBwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse;    // [B][Hq][N]
    const float* delta;  // [B][Hq][N]
    void* dq;
    void* dk;
    void* dv;
    float* dq_part;      // [B][Hq][n_global][n_key_chunks][D] float32 partials
    float* dkv_part;     // [B][Hkv][n_global][n_row_chunks][2][D] float32 partials
    int B, Hq, Hkv, N, group;
    int wl, wr, dil, causal;
    float scale, scale_log2;
    int n_global;
    int row_tiles;        // tiles of kGlobalBwdItems global rows
    int key_chunk, n_key_chunks;   // key split of the global-row dq pass
    int key_tiles;        // tiles of kGlobalBwdItems global keys
    int row_chunk, n_row_chunks;   // row split of the global-key dk/dv pass
    int n_row_tiles_all;  // 64-row tiles of all N rows
    int n_key_tiles_all;  // 64-key tiles of all N keys
    int fused;            // kGlobalColsDqFused | kGlobalRowsDkdvFused: passes the band
                          // kernels already did (their launches are skipped)
    int32_t gpos[SWA_MAX_GLOBAL];  // sorted, unique
};
constexpr int kGlobalColsDqFused = 1;    // dq of other rows from global keys
constexpr int kGlobalRowsDkdvFused = 2;  // dk, dv of every key from global rows

struct DecodeParams {
    const void* q;
    const void* kcache;
    const void* vcache;
    const int32_t* ring_head;
    const int32_t* cache_len;
    float* partials;   // [B][Hq][splits][D+4]
    // bf16 kernel with splits == 1: the rows are written here directly
    // ([B][Hq][D], lse [B][Hq] or null) and no partials are made
    void* out;
    float* lse;
    int B, Hq, Hkv, W, group;
    int splits;        // partials per row: the ring splits, plus (f32 kernel) one
                       // for the sinks; the bf16 kernel walks the sinks in split 0
    int ring_splits;   // splits over the ring's W slots
    int slots_per_split;
    float scale_log2;
    // attention-sink entries [B][Hkv][n_sink][D] beside the ring (n_sink = 0: none)
    const void* ksink;
    const void* vsink;
    int n_sink;
    // paged cache (paged kernels only): kcache/vcache are the page pool
    // [n_pages][Hkv][P][D], P = 1 << page_shift; position t of sequence b is in
    // page block_table[b * nb + (t >> page_shift) % nb]; seq_len[b] tokens so far
    const int32_t* block_table;
    const int32_t* seq_len;
    int n_pages, page_shift, nb;
};

struct CombineParams {
    const float* partials;  // [rows][splits][D+4]
    void* out;
    float* lse;             // may be null
    int rows, splits;
    int mode;               // 0: decode rows (b*Hq + h); 1: global rows of a forward
    int B, Hq, N, n_global;
    int32_t gpos[SWA_MAX_GLOBAL];
};

// Workgroup shape of a forward kernel for a GQA group size: query heads per
// workgroup, query positions (of one residue class) per workgroup, and global
// query rows per workgroup in the global-row pass.
struct FwdShape {
    int hpw;
    int bmq;
    int grows_rows;
};
FwdShape fwd_bf16_shape(int group);
FwdShape fwd_f32_shape(int group);

// Launchers (return hipError_t of the launch).
hipError_t launch_fwd_bf16(const FwdParams& p, int D, hipStream_t s);
// Two-group (phase-offset) bf16 forward: D = 128, four query heads per
// workgroup, band only (no global tokens, no ring).  launch_fwd_bf16 uses it
// where it applies.
bool fwd_pp_applies(const FwdParams& p, int D);
hipError_t launch_fwd_pp(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int D, hipStream_t s);
FwdShape bwd_bf16_dq_shape(int group);
int bwd_bf16_dkdv_keys();
FwdShape bwd_f32_dq_shape(int group);
int bwd_f32_dkdv_keys();
hipError_t launch_bwd_delta(const BwdParams& p, int D, hipStream_t s);   // float32
hipError_t launch_bwd_bf16(const BwdParams& p, int D, hipStream_t s);
hipError_t launch_bwd_f32(const BwdParams& p, int D, hipStream_t s);
hipError_t launch_bwd_global(const GlobalBwdParams& g, int D, int dtype, hipStream_t s);
hipError_t launch_kv_append(void* kc, void* vc, const void* kn, const void* vn,
                            int32_t* head, int32_t* len, int B, int Hkv, int W, int D,
                            int elem_bytes, hipStream_t s);
hipError_t launch_kv_append_chunk(void* kc, void* vc, const void* k, const void* v,
                                  int32_t* head, int32_t* len, int B, int Hkv, int W, int n,
                                  int D, int elem_bytes, hipStream_t s);
hipError_t launch_kv_append_paged(void* kpool, void* vpool, const void* k, const void* v,
                                  const int32_t* block_table, int32_t* seq_len, int B, int Hkv,
                                  int n_pages, int page_shift, int nb, int W, int n, int D,
                                  int elem_bytes, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeParams& p, int D, bool paged, hipStream_t s);
hipError_t launch_decode_f32(const DecodeParams& p, int D, bool paged, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, int D, int dtype, hipStream_t s);

#ifdef SWA_DEBUG
// Debug build: read (and optionally clear) the failed-check counter of one
// kernel source file on the current device.
hipError_t debug_counter_fwd_bf16(unsigned* value, bool reset);
hipError_t debug_counter_fwd_pp(unsigned* value, bool reset);
hipError_t debug_counter_fwd_f32(unsigned* value, bool reset);
hipError_t debug_counter_bwd_bf16(unsigned* value, bool reset);
hipError_t debug_counter_decode(unsigned* value, bool reset);
#endif

}  // namespace swa
