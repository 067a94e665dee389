/*
 * swa.h -- C ABI of libswa.so: sliding-window attention for AMD MI355X (gfx950).
 *
 * The operation (bmjup.com, "Sliding window attention", section "core
 * principle", mathematical form): for every query position i,
 *     y_i = sum_{j in S(i)} softmax_j(scale * q_i . k_j) v_j
 * where S(i) is the window around i, truncated at the sequence edges.
 *
 * Window parameters (explicit left/right extents counted in dilated steps):
 *   Band(i) = { i + t*dilation : -win_left <= t <= win_right } intersected with [0, N)
 *   - causal window of W keys, [i-W+1, i]:     win_left = W-1, win_right = 0
 *     (bmjup.com, "bidirectional vs unidirectional sliding window": a causal
 *      query sees only keys to its left; aiqz.cc "Python demo": the last
 *      window_size keys, the current one included)
 *   - bidirectional odd W, [i-(W-1)/2, i+(W-1)/2]: win_left = win_right = (W-1)/2
 *   - dilated windows i +- t*d (mhpn.cn "Dilated sliding window", section 2
 *     "structure comparison"): dilation = d
 * The call is causal exactly when win_right == 0.
 *
 * Global tokens (aiqz.cc, "global attention tokens"; mhpn.cn, section 3,
 * "attention sink"): a global position g is seen by every query (by queries
 * i >= g when causal), and a global query row attends to every key (keys
 * j <= i when causal).  S(i) is a set: a global key inside the band counts
 * once.
 *
 * Decode (intelliparadigm.com, section 3.1 "cache mechanism", RingBuffer:
 * write buffer[idx % size], then idx += 1; aiqz.cc, "inference optimisation":
 * the cache keeps only the last W entries): a ring of W slots per sequence.
 * ring_head[b] is the next slot to write; cache_len[b] (<= W) counts valid
 * entries.  After an append, the valid slots of sequence b are
 *     { (ring_head[b] - 1 - a) mod W : 0 <= a < cache_len[b] }.
 *
 * Conventions for every entry point:
 *   - Layouts are row-major and contiguous:
 *       q, out        [B, N, Hq, D]       (batch, sequence, heads, head dim)
 *       k, v          [B, N, Hkv, D]
 *       lse           [B, Hq, N]  float32, natural log of the softmax partition
 *                     function of the scaled scores
 *       decode q, out [B, Hq, D];  decode lse [B, Hq] float32
 *       kcache,vcache [B, Hkv, W, D]
 *     Query head h reads kv head h / (Hq / Hkv) (grouped-query attention).
 *   - Element type of q, k, v, out, kcache, vcache, k_new, v_new: `dtype`
 *     (SWA_F32 or SWA_BF16).  Accumulation is float32.  In bf16 the softmax
 *     weights are rounded to bf16 (nearest even) before the weighted sum of v.
 *   - D must be 64 or 128.
 *   - `scale` (every entry point that takes one) is the softmax temperature
 *     that multiplies q.k: it must be positive and finite (so must scale *
 *     log2(e)); zero, negative, infinite or NaN scales give SWA_ERR_ARG.  The
 *     scaled scores themselves must stay within float32 range.
 *   - Device pointers are caller-owned device memory.  The library allocates
 *     nothing and keeps no state between calls; all work is enqueued on
 *     `stream` (0 = the null stream) and nothing synchronises the host.
 *   - Return value: SWA_OK, or a negative status.  Argument errors are found
 *     before anything is enqueued.  SWA_ERR_HIP reports a launch failure
 *     (hipGetLastError); faults during execution surface at the caller's next
 *     synchronisation.  Calls on one stream are ordered; the library is
 *     thread-safe (stateless).
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SWA_F32 = 0, SWA_BF16 = 1 } swa_dtype;

enum {
    SWA_OK = 0,
    SWA_ERR_ARG = -1,          /* null pointer, bad size, bad window, bad global index */
    SWA_ERR_UNSUPPORTED = -2,  /* D not in {64, 128}, unknown dtype, too many globals */
    SWA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
    SWA_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed */
};

/* Largest number of distinct global positions one swa_fwd call accepts. */
#define SWA_MAX_GLOBAL 256

/* Longest sequence one swa_fwd call accepts (2^28 positions). */
#define SWA_MAX_N (1 << 28)

/*
 * swa_fwd: sliding-window attention over whole sequences (prefill / encoder).
 *
 *   q, k, v     device, inputs as above (read only)
 *   out         device, [B, N, Hq, D] of `dtype` (written)
 *   lse         device, [B, Hq, N] float32 (written); may be NULL to skip it
 *   B, Hq, Hkv, N, D   sizes; Hq % Hkv == 0
 *   win_left, win_right >= 0, dilation >= 1.  Windows wider than the sequence
 *               are clipped, not rejected.
 *   global_idx  HOST array of n_global positions in [0, N) (may hold
 *               duplicates, any order); NULL when n_global == 0.  At most
 *               SWA_MAX_GLOBAL distinct positions.  The array is read during
 *               the call only.
 *   scale       multiplier of q.k (1/sqrt(D) for the usual softmax_scale);
 *               positive and finite
 *   workspace   device scratch of at least swa_fwd_workspace_size(...) bytes,
 *               caller-owned, contents on entry irrelevant; used only when
 *               there are global positions (partial results of the global
 *               query rows, which are split over the keys and merged).  Two
 *               calls in flight at once must not share it.
 *
 * Errors: SWA_ERR_ARG for null q/k/v/out, non-positive sizes, N > SWA_MAX_N,
 * Hq % Hkv != 0,
 * negative windows, dilation < 1, a global index outside [0, N), n_global < 0
 * or global_idx NULL with n_global > 0, or a scale that is not positive and
 * finite; SWA_ERR_UNSUPPORTED for D not in
 * {64,128}, an unknown dtype or more than SWA_MAX_GLOBAL distinct globals;
 * SWA_ERR_WORKSPACE when globals are present and the workspace is NULL or
 * smaller than swa_fwd_workspace_size(); SWA_ERR_HIP if a launch fails.
 */
int swa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
            int B, int Hq, int Hkv, int N, int D,
            int win_left, int win_right, int dilation,
            const int32_t* global_idx, int n_global,
            float scale, int dtype,
            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace swa_fwd needs (0 when n_global == 0, in which case
 * workspace may be NULL).  n_global may count duplicates; 0 on bad sizes. */
size_t swa_fwd_workspace_size(int B, int Hq, int N, int D, int n_global);

/*
 * swa_kv_append: write one new token per sequence into the ring (the
 * RingBuffer append of intelliparadigm.com, section 3.1), on the device:
 *   kcache[b, :, ring_head[b], :] = k_new[b];  vcache likewise;
 *   ring_head[b] = (ring_head[b] + 1) % W;  cache_len[b] = min(cache_len[b] + 1, W)
 *
 *   kcache, vcache   device, [B, Hkv, W, D] of `dtype` (updated in place)
 *   k_new, v_new     device, [B, Hkv, D] of `dtype`
 *   ring_head, cache_len   device int32 [B] (updated in place); on entry
 *                    0 <= ring_head < W and 0 <= cache_len <= W.  Values out
 *                    of range are the caller's error; the kernels clamp them
 *                    into range so that no access leaves the ring.
 *
 * Errors: SWA_ERR_ARG for null pointers or non-positive sizes;
 * SWA_ERR_UNSUPPORTED for D or dtype; SWA_ERR_HIP if the launch fails.
 */
int swa_kv_append(void* kcache, void* vcache, const void* k_new, const void* v_new,
                  int32_t* ring_head, int32_t* cache_len,
                  int B, int Hkv, int W, int D, int dtype, hipStream_t stream);

/*
 * swa_kv_append_chunk: append n tokens per sequence to the ring at once, with
 * the same result as n calls of swa_kv_append in token order
 * (intelliparadigm.com, section 3.1, RingBuffer; aiqz.cc, "inference
 * optimisation": the cache rolls and keeps the last W entries).  Token t of
 * the chunk goes to slot (ring_head[b] + t) % W; when n > W only the last W
 * tokens are written.  Then ring_head[b] = (ring_head[b] + n) % W and
 * cache_len[b] = min(cache_len[b] + n, W).  Used to hand a prefilled prompt
 * (or one chunk of it) over to decode.
 *
 *   kcache, vcache   device, [B, Hkv, W, D] of `dtype` (updated in place)
 *   k, v             device, [B, n, Hkv, D] of `dtype` (the layout of swa_fwd's k, v);
 *                    may be NULL when n == 0
 *   ring_head, cache_len   device int32 [B], as for swa_kv_append
 *   n                tokens per sequence, 0 <= n <= SWA_MAX_N (0: nothing to do)
 *
 * Errors: as swa_kv_append (k, v may be NULL only when n == 0), plus
 * SWA_ERR_ARG for n < 0 or n or W above SWA_MAX_N.
 */
int swa_kv_append_chunk(void* kcache, void* vcache, const void* k, const void* v,
                        int32_t* ring_head, int32_t* cache_len,
                        int B, int Hkv, int W, int n, int D, int dtype, hipStream_t stream);

/*
 * swa_fwd_cached: causal sliding-window attention of a prompt chunk that
 * follows the tokens held in the ring (streaming prefill: aiqz.cc, "inference
 * optimisation", third strategy; bmjup.com, Q&A "training vs inference").
 * Let P be the position of chunk token 0; the ring of sequence b holds the
 * cache_len[b] tokens before it, the one of age a (0 = newest, position
 * P - 1 - a) in slot (ring_head[b] - 1 - a) mod W.  Query t of the chunk
 * attends to every held key at positions P + t - win_left .. P + t:
 *   ring entries of age a < cache_len[b] with a <= win_left - 1 - t, and
 *   chunk tokens j with max(0, t - win_left) <= j <= t.
 * The ring is read only; append the chunk afterwards (swa_kv_append_chunk)
 * to continue with the next chunk or with decode.  No dilation and no global
 * tokens on this path.
 *
 *   q, out      device, [B, n, Hq, D] of `dtype`
 *   k, v        device, [B, n, Hkv, D] of `dtype` (the chunk's own keys/values)
 *   kcache, vcache, ring_head, cache_len   device, as for swa_kv_append
 *   lse         device, [B, Hq, n] float32 (may be NULL)
 *   n           chunk length, 1 <= n <= SWA_MAX_N
 *   win_left    keys before the query, 0 <= win_left <= W (older keys could
 *               have left the ring)
 *   scale       multiplier of q.k (1/sqrt(D) for the usual scaling)
 *
 * Errors: SWA_ERR_ARG for null pointers (lse excepted), non-positive sizes,
 * n or W above SWA_MAX_N, Hq % Hkv != 0, win_left < 0 or win_left > W, or a
 * scale that is not positive and finite; SWA_ERR_UNSUPPORTED for D or dtype;
 * SWA_ERR_HIP if a launch fails.
 */
int swa_fwd_cached(const void* q, const void* k, const void* v,
                   const void* kcache, const void* vcache,
                   const int32_t* ring_head, const int32_t* cache_len,
                   void* out, float* lse,
                   int B, int Hq, int Hkv, int n, int W, int D,
                   int win_left, float scale, int dtype, hipStream_t stream);

/*
 * swa_decode: one query token per sequence attends over the valid ring slots
 * (aiqz.cc, "Python demo" and "inference optimisation": the last cache_len
 * entries, the newest included).  Call it after swa_kv_append for the step.
 *
 *   q           device, [B, Hq, D] of `dtype`
 *   kcache, vcache, ring_head, cache_len   device, as for swa_kv_append (read
 *               only).  A sequence with cache_len == 0 gets out = 0 and
 *               lse = -inf.
 *   out         device, [B, Hq, D] of `dtype`;  lse device [B, Hq] float32
 *               (may be NULL)
 *   workspace   device scratch of at least swa_decode_workspace_size(B, Hq, W, D)
 *               bytes, owned by the caller; its contents on entry do not
 *               matter.  It holds split partials; a bf16 launch whose rings
 *               each take one slot range writes the rows directly and leaves
 *               it untouched.  Two calls in flight at once must not share it.
 *
 * Errors: as swa_kv_append, plus SWA_ERR_ARG for Hq % Hkv != 0, a scale that
 * is not positive and finite, or sizes whose launch grid would pass 2^31 - 1
 * workgroups, and SWA_ERR_WORKSPACE when the workspace is NULL or too small.
 */
int swa_decode(const void* q, const void* kcache, const void* vcache,
               const int32_t* ring_head, const int32_t* cache_len,
               void* out, float* lse,
               int B, int Hq, int Hkv, int W, int D, float scale,
               void* workspace, size_t workspace_bytes, int dtype, hipStream_t stream);

/* Bytes of device workspace swa_decode needs for these sizes (0 on bad sizes). */
size_t swa_decode_workspace_size(int B, int Hq, int W, int D);

/*
 * swa_decode_noalloc: swa_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (minus the
 * workspace), same kernels and the same result bit for bit.  The split
 * partials live in a device array inside the library,
 * SWA_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on a GPU until
 * the process ends; the call itself allocates nothing.
 *
 * Every call on one GPU shares that GPU's array: two calls that overlap in
 * time on one GPU (different streams, or host threads) race and give wrong
 * results; calls on one stream are ordered and safe.  The array needs no
 * clearing (each call writes every record it reads).  `stream` must belong to
 * the current device.
 *
 * A launch needs B * Hq * splits * (D + 4) * 4 bytes of it, where splits is
 * the number of slot ranges each ring is cut into (the bf16 kernel with one
 * range per ring, e.g. 64 sequences x 8 kv heads, needs none).  With the
 * 16 MiB array, 64 sequences x 32 heads at D = 128 fit up to 15 ranges.
 *
 * Errors: as swa_decode, except SWA_ERR_WORKSPACE means the launch needs more
 * than SWA_NOALLOC_SCRATCH_BYTES; SWA_ERR_HIP also if the array's device
 * address cannot be found.
 */
#define SWA_NOALLOC_SCRATCH_BYTES (16u << 20)
int swa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                       const int32_t* ring_head, const int32_t* cache_len,
                       void* out, float* lse,
                       int B, int Hq, int Hkv, int W, int D, float scale,
                       int dtype, hipStream_t stream);

/*
 * swa_decode_sinks: swa_decode plus n_sink attention-sink entries that stay
 * visible to every step and are never evicted (mhpn.cn "Dilated sliding
 * window", section 3: the first tokens kept as attention-sink anchors; aiqz.cc,
 * "global attention tokens").  The sink buffers hold the first n_sink tokens
 * of each sequence; those tokens do not enter the ring, which holds the tokens
 * after them.  Each query attends the valid ring slots and all sink entries;
 * the result equals the causal window-W forward with global positions
 * 0..n_sink-1 at the decode row (W = ring size, window W keys).
 *
 *   ksink, vsink  device, [B, Hkv, n_sink, D] of `dtype` (read only); may be
 *                 NULL when n_sink == 0.  Filling them: swa_kv_append_chunk on
 *                 a ring of n_sink slots starting at ring_head = cache_len = 0
 *                 puts token t of the chunk in slot t.
 *   n_sink        0 <= n_sink <= SWA_MAX_N.  The bf16 kernel walks the sink
 *                 entries in the first slot range of each (b, kv head), the
 *                 fp32 kernel in a range of their own; either way they should
 *                 stay few next to W.
 *   workspace     at least swa_decode_sinks_workspace_size(B, Hq, W, D, n_sink)
 *                 bytes.
 *   Everything else as for swa_decode (which is this call with n_sink == 0).
 *   A sequence with cache_len == 0 and n_sink == 0 gets out = 0, lse = -inf.
 *
 * Errors: as swa_decode, plus SWA_ERR_ARG for n_sink < 0, n_sink > SWA_MAX_N
 * or NULL sink buffers with n_sink > 0.
 */
int swa_decode_sinks(const void* q, const void* kcache, const void* vcache,
                     const int32_t* ring_head, const int32_t* cache_len,
                     const void* ksink, const void* vsink, int n_sink,
                     void* out, float* lse,
                     int B, int Hq, int Hkv, int W, int D, float scale,
                     void* workspace, size_t workspace_bytes, int dtype, hipStream_t stream);

/* Bytes of device workspace swa_decode_sinks needs (0 on bad sizes). */
size_t swa_decode_sinks_workspace_size(int B, int Hq, int W, int D, int n_sink);

/*
 * Paged window cache (mhpn.cn "Dilated sliding window", section 4, KV-cache
 * management: entries that left the window are freed page by page;
 * intelliparadigm.com, section 6: a pre-allocated memory pool, cache updates
 * without copies).  Keys and values live in a pool of pages shared by all
 * sequences:
 *   kpool, vpool   device, [n_pages, Hkv, P, D] of `dtype`; a page holds P
 *                  consecutive positions (P = page_size, a power of two) of
 *                  one sequence for every kv head
 *   block_table    device int32 [B, nb]: position t of sequence b is in page
 *                  block_table[b*nb + (t / P) % nb], slot t % P.  nb*P must be
 *                  at least W + P - 1, so that the blocks meeting the last W
 *                  positions sit in distinct entries.
 *   seq_len        device int32 [B]: tokens appended so far (positions
 *                  0 .. seq_len[b] - 1)
 * The caller owns the pool and the table and decides which page each entry
 * points to.  Before an append it points the entries of the blocks the new
 * positions fall in at pages; an entry whose block holds no position of the
 * last W may be re-pointed, its page going back to the pool (eviction).
 * Page ids out of [0, n_pages) are clamped into the pool (no fault; the
 * result is then meaningless).
 */

/*
 * swa_kv_append_paged: append n tokens per sequence, k, v [B, n, Hkv, D], at
 * positions seq_len[b] .. seq_len[b] + n - 1; only the last min(n, W) are
 * written (older ones are outside every later window).  Then seq_len[b] += n.
 * n = 1 is the decode-step append; n > 1 hands a prefilled chunk over.
 *
 * Errors: SWA_ERR_ARG for null pointers (k, v may be NULL when n == 0),
 * non-positive sizes, n < 0, n or W above SWA_MAX_N, page_size not a power of
 * two up to 2^20, or nb*page_size < W + page_size - 1; SWA_ERR_UNSUPPORTED for
 * D or dtype; SWA_ERR_HIP if a launch fails.
 */
int swa_kv_append_paged(void* kpool, void* vpool, const void* k, const void* v,
                        const int32_t* block_table, int32_t* seq_len,
                        int B, int Hkv, int n_pages, int page_size, int nb, int W, int n,
                        int D, int dtype, hipStream_t stream);

/*
 * swa_decode_paged: one query token per sequence, q [B, Hq, D], attends the
 * last min(seq_len[b], W) positions (the newest included) through the block
 * table; the same result as swa_decode on a W-slot ring fed the same tokens.
 *   out [B, Hq, D] of `dtype`; lse [B, Hq] float32 (may be NULL);
 *   workspace of at least swa_decode_workspace_size(B, Hq, W, D) bytes.
 * A sequence with seq_len == 0 gets out = 0, lse = -inf.
 *
 * Errors: as swa_kv_append_paged, plus SWA_ERR_ARG for Hq % Hkv != 0 or a
 * scale that is not positive and finite, and SWA_ERR_WORKSPACE when the
 * workspace is NULL or too small.
 */
int swa_decode_paged(const void* q, const void* kpool, const void* vpool,
                     const int32_t* block_table, const int32_t* seq_len,
                     void* out, float* lse,
                     int B, int Hq, int Hkv, int n_pages, int page_size, int nb, int W, int D,
                     float scale, void* workspace, size_t workspace_bytes, int dtype,
                     hipStream_t stream);

/*
 * swa_bwd: gradients of swa_fwd (training use: bmjup.com "Sliding window
 * attention", Q&A on training vs inference; intelliparadigm.com section 5.1,
 * blocked and mixed-precision training).  For the upstream gradient dout of
 * out, with P_ij the forward's attention weights over S(i) and
 * dP_ij = dout_i . v_j:
 *   dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
 *   dq_i = scale sum_j dS_ij k_j;  dk_j = scale sum_i dS_ij q_i;  dv_j = sum_i P_ij dout_i
 * (a kv head collects the terms of every query head of its group).  P is
 * rebuilt from the forward's lse, so out and lse must come from swa_fwd with
 * the same arguments.  In bf16, P and dS are rounded to bf16 before their
 * products, as the forward rounds its weights.
 *
 *   q, k, v, out, dout   device, layouts and dtype of swa_fwd (dout like out)
 *   lse                  device, [B, Hq, N] float32 from swa_fwd (required)
 *   dq                   device, [B, N, Hq, D] of `dtype` (written)
 *   dk, dv               device, [B, N, Hkv, D] of `dtype` (written; keys no
 *                        query attends get 0)
 *   win_left, win_right, dilation, scale   as for swa_fwd
 *   global_idx, n_global as for swa_fwd (host array).  Global rows take the
 *                        terms of every key they attend, every row the terms
 *                        of the global keys it attends (aiqz.cc "Sliding
 *                        window attention: Mistral", section "global attention
 *                        tokens").  The pairs outside the band are summed in
 *                        float32.  In bf16 the pairs of ordinary rows with
 *                        global keys join their row's dq before its one
 *                        rounding, and at D = 64 so do the global rows'
 *                        pairs with every key in that key's dk, dv; the
 *                        other such terms (a global row's dq, a global key's
 *                        dk and dv, and float32 or D = 128 where no band pass
 *                        takes them) are added to the band's result, one more
 *                        rounding of those rows in bf16.  Work split over key
 *                        or row chunks writes one float32 partial per chunk,
 *                        summed in chunk order: no atomics, and the same call
 *                        gives the same bits every time.
 *   workspace            device scratch of swa_bwd_workspace_size() bytes
 *                        (per-row dout . out; with global tokens also the
 *                        float32 partials of their rows and keys); two calls
 *                        in flight at once must not share it
 *
 * Errors: as swa_fwd (with lse, dout, dq, dk, dv required), plus
 * SWA_ERR_WORKSPACE for a missing or short workspace.
 */
int swa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
            const void* dout, void* dq, void* dk, void* dv,
            int B, int Hq, int Hkv, int N, int D,
            int win_left, int win_right, int dilation,
            const int32_t* global_idx, int n_global,
            float scale, int dtype,
            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace swa_bwd needs for n_global global tokens (the
 * count passed to swa_bwd, duplicates included, is enough); 0 on bad sizes. */
size_t swa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int D, int n_global);

/* A static, human-readable description of a status code. */
const char* swa_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int swa_version(void);

/* Index-contract checks of the debug build (libswa_debug.so, compiled with
 * SWA_DEBUG; not an operation of the method).  In that build the kernels check
 * every global row they read or write against its tensor, ring slots and
 * sink entries against the cache, LDS tile offsets against the tile, and the
 * device-side state they are handed (ring_head, cache_len, seq_len, block_table
 * entries) against its documented range before clamping it; a failed check is
 * counted, once per thread that evaluates it, and never faults.  That build
 * also adds workgroup barriers that run overlapped phases one after another
 * and waits on every tile copy as soon as it is issued: its results match the
 * release build's bit for bit unless a wait or barrier is missing there.
 * This call waits for all work on the current device (hipDeviceSynchronize),
 * stores the number of failed checks counted on that device since the last
 * reset in *count (if count is non-null), and clears the counters when reset
 * is non-zero.  Returns SWA_OK, SWA_ERR_HIP if a HIP call fails, and
 * SWA_ERR_UNSUPPORTED in the release build (count is left unchanged). */
int swa_debug_violations(unsigned long long* count, int reset);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
