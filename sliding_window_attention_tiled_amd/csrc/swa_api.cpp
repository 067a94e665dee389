// swa_api.cpp -- the C ABI of libswa.so (declared in include/swa.h): argument
// validation, normalisation of the global set, work planning and launches.
// Nothing here allocates device memory or synchronises the host.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include <hip/hip_runtime.h>

#include "swa_kernels.h"

namespace {

using swa::CombineParams;
using swa::DecodeParams;
using swa::FwdParams;

// Longest sequence accepted: keeps every position, window offset and the
// kernels' out-of-window sentinel (-2^30) within 32-bit integer range.
constexpr int kMaxN = SWA_MAX_N;
constexpr float kLog2e = 1.4426950408889634f;

bool supported_d(int D) { return D == 64 || D == 128; }
// The kernels mask a key by setting its raw score to -inf before the multiply
// by scale * log2(e) and take the running max on raw scores: both need a
// positive, finite multiplier.  (scale <= 0 has no meaning for a softmax
// temperature; NaN fails the comparison.)
bool valid_scale(float scale) { return scale > 0.f && std::isfinite(scale * kLog2e); }
bool known_dtype(int dt) { return dt == SWA_F32 || dt == SWA_BF16; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Key chunking of global query rows: at most 32 chunks, each a multiple of 64 keys.
void global_chunks(int N, int* chunk, int* nchunks) {
    int64_t nc = std::min<int64_t>(32, std::max<int64_t>(1, cdiv(N, 512)));
    int64_t ck = cdiv(cdiv(N, nc), 64) * 64;
    *chunk = (int)ck;
    *nchunks = (int)cdiv(N, ck);
}

// The global positions sorted and deduplicated; SWA_ERR_ARG for a position
// outside [0, N), SWA_ERR_UNSUPPORTED for more than SWA_MAX_GLOBAL of them.
int normalize_globals(const int32_t* global_idx, int n_global, int N, std::vector<int32_t>& g) {
    g.assign(global_idx, global_idx + n_global);
    for (int32_t x : g)
        if (x < 0 || x >= N) return SWA_ERR_ARG;
    std::sort(g.begin(), g.end());
    g.erase(std::unique(g.begin(), g.end()), g.end());
    return (int)g.size() > SWA_MAX_GLOBAL ? SWA_ERR_UNSUPPORTED : SWA_OK;
}

// Splits of a decode ring, each a multiple of 128 slots.  The bf16 kernel runs
// one 4-wave workgroup per (sequence, kv head, 16-head block, split) and two of
// them are resident per CU at D = 128: about 512 workgroups fill the 256 CUs
// once, and fewer, longer splits start and drain fewer workgroups and leave
// fewer partials to merge (none with one split).  The f32 kernel runs one
// wave per (sequence, query head, split) and aims at 8192 waves.
constexpr int64_t kDecodeWorkgroups = 512;
constexpr int64_t kDecodeWavesF32 = 8192;

void decode_splits(int dtype, int B, int Hq, int Hkv, int W, int* splits, int* per_split) {
    const int64_t units = dtype == SWA_BF16 ? (int64_t)B * Hkv * cdiv(Hq / Hkv, 16)
                                            : (int64_t)B * Hq;
    const int64_t target = dtype == SWA_BF16 ? kDecodeWorkgroups : kDecodeWavesF32;
    int64_t sp = std::max<int64_t>(1, cdiv(target, units));
    sp = std::min<int64_t>(sp, std::max<int64_t>(1, W / 128));
    int64_t ps = cdiv(cdiv(W, sp), 128) * 128;
    *per_split = (int)ps;
    *splits = (int)cdiv(W, ps);
}

// Partials per row that a decode of these sizes can use, for either dtype and
// any Hkv dividing Hq: the bf16 kernel makes the most splits at Hkv = 1 (the
// fewest workgroup units), the f32 kernel adds one split for the sinks.
int decode_max_splits(int B, int Hq, int W, int n_sink) {
    int sb, sf, per;
    decode_splits(SWA_BF16, B, Hq, 1, W, &sb, &per);
    decode_splits(SWA_F32, B, Hq, Hq, W, &sf, &per);
    return std::max(sb, sf + (n_sink > 0 ? 1 : 0));
}

// Band work decomposition of a forward launch (p.B, Hkv, group, N, dil set).
// False when the grid would not fit in 32 bits.
bool plan_band_shape(FwdParams& p, const swa::FwdShape& shape) {
    p.qd = p.N / p.dil;
    p.rem = p.N % p.dil;
    p.hpw = shape.hpw;
    p.bmq = shape.bmq;
    p.head_groups = p.group / p.hpw;
    p.tiles_long = (int)cdiv(p.qd + 1, p.bmq);
    p.tiles_short = (int)cdiv(p.qd, p.bmq);
    const int64_t per_slab =
        (int64_t)p.rem * p.tiles_long + (int64_t)(p.dil - p.rem) * p.tiles_short;
    const int64_t blocks = (int64_t)p.B * p.Hkv * p.head_groups * per_slab;
    if (per_slab > INT32_MAX || blocks > INT32_MAX) return false;
    p.tiles_per_slab = (int)per_slab;
    p.n_blocks = (int)blocks;
    return true;
}

bool plan_band(FwdParams& p, int dtype, swa::FwdShape* shape_out) {
    *shape_out = dtype == SWA_BF16 ? swa::fwd_bf16_shape(p.group) : swa::fwd_f32_shape(p.group);
    return plan_band_shape(p, *shape_out);
}

// Merges the split partials of a decode launch into out / lse.
int combine_decode(const DecodeParams& p, void* out, float* lse, int D, int dtype,
                   hipStream_t stream) {
    CombineParams c;
    std::memset(&c, 0, sizeof c);
    c.partials = p.partials;
    c.out = out;
    c.lse = lse;
    c.rows = p.B * p.Hq;
    c.splits = p.splits;
    c.mode = 0;
    c.B = p.B;
    c.Hq = p.Hq;
    return swa::launch_combine(c, D, dtype, stream) == hipSuccess ? SWA_OK : SWA_ERR_HIP;
}

// Split decode launch, then the merge of its partials.  The bf16 kernel walks
// sink entries within split 0 and, with a single split, writes the rows
// itself; the f32 kernel gives the sinks a split of their own.
int run_decode(DecodeParams& p, void* out, float* lse, int D, int dtype, bool paged,
               hipStream_t stream) {
    const bool bf16 = dtype == SWA_BF16;
    p.splits = p.ring_splits + (!bf16 && !paged && p.n_sink > 0 ? 1 : 0);
    // grids: bf16 one workgroup per (b, kv head, 16-head block, split), float32
    // one per (b, query head, split); the merge one per (b, query head)
    const int64_t grid = bf16 ? (int64_t)p.B * p.Hkv * cdiv(p.group, 16) * p.splits
                              : (int64_t)p.B * p.Hq * p.splits;
    if (grid > INT32_MAX || (int64_t)p.B * p.Hq > INT32_MAX) return SWA_ERR_ARG;
    if (bf16 && p.splits == 1) {
        p.out = out;
        p.lse = lse;
    }
    hipError_t e = bf16 ? swa::launch_decode_bf16(p, D, paged, stream)
                        : swa::launch_decode_f32(p, D, paged, stream);
    if (e != hipSuccess) return SWA_ERR_HIP;
    if (p.out != nullptr) return SWA_OK;
    return combine_decode(p, out, lse, D, dtype, stream);
}

// Validates the arguments of a ring decode (with n_sink sink entries) and
// fills its launch parameters, the split plan included; the caller supplies
// the partials buffer.
int plan_ring_decode(DecodeParams& p, const void* q, const void* kcache, const void* vcache,
                     const int32_t* ring_head, const int32_t* cache_len, const void* ksink,
                     const void* vsink, int n_sink, const void* out, int B, int Hq, int Hkv,
                     int W, int D, float scale, int dtype) {
    if (!q || !kcache || !vcache || !ring_head || !cache_len || !out) return SWA_ERR_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || W <= 0 || D <= 0 || Hq % Hkv != 0) return SWA_ERR_ARG;
    if (n_sink < 0 || n_sink > kMaxN || (n_sink > 0 && (!ksink || !vsink))) return SWA_ERR_ARG;
    if (!valid_scale(scale)) return SWA_ERR_ARG;
    if (!supported_d(D) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.kcache = kcache;
    p.vcache = vcache;
    p.ring_head = ring_head;
    p.cache_len = cache_len;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.W = W;
    p.group = Hq / Hkv;
    p.scale_log2 = scale * kLog2e;
    decode_splits(dtype, B, Hq, Hkv, W, &p.ring_splits, &p.slots_per_split);
    p.ksink = ksink;
    p.vsink = vsink;
    p.n_sink = n_sink;
    return SWA_OK;
}

// log2 of a power of two in [1, 2^20], else -1
int page_shift_of(int P) {
    for (int sh = 0; sh <= 20; sh++)
        if (P == (1 << sh)) return sh;
    return -1;
}

}  // namespace

extern "C" {

const char* swa_status_string(int status) {
    switch (status) {
        case SWA_OK: return "success";
        case SWA_ERR_ARG: return "invalid argument";
        case SWA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or global count";
        case SWA_ERR_WORKSPACE: return "workspace missing or too small";
        case SWA_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int swa_version(void) { return 100; }

int swa_debug_violations(unsigned long long* count, int reset) {
#ifdef SWA_DEBUG
    if (hipDeviceSynchronize() != hipSuccess) return SWA_ERR_HIP;
    hipError_t (*const readers[])(unsigned*, bool) = {
        swa::debug_counter_fwd_bf16, swa::debug_counter_fwd_pp, swa::debug_counter_fwd_f32,
        swa::debug_counter_bwd_bf16, swa::debug_counter_decode};
    unsigned long long total = 0;
    for (auto read : readers) {
        unsigned v = 0;
        if (read(&v, reset != 0) != hipSuccess) return SWA_ERR_HIP;
        total += v;
    }
    if (count != nullptr) *count = total;
    return SWA_OK;
#else
    (void)count;
    (void)reset;
    return SWA_ERR_UNSUPPORTED;
#endif
}

size_t swa_fwd_workspace_size(int B, int Hq, int N, int D, int n_global) {
    if (B <= 0 || Hq <= 0 || N <= 0 || N > kMaxN || !supported_d(D) || n_global < 0) return 0;
    if (n_global == 0) return 0;
    const int ng = std::min(n_global, SWA_MAX_GLOBAL);
    int chunk, nchunks;
    global_chunks(N, &chunk, &nchunks);
    return (size_t)B * Hq * ng * nchunks * swa::partial_floats(D) * sizeof(float);
}

int swa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
            int Hkv, int N, int D, int win_left, int win_right, int dilation,
            const int32_t* global_idx, int n_global, float scale, int dtype, void* workspace,
            size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !out) return SWA_ERR_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || N > kMaxN || D <= 0) return SWA_ERR_ARG;
    if (Hq % Hkv != 0) return SWA_ERR_ARG;
    if (win_left < 0 || win_right < 0 || dilation < 1) return SWA_ERR_ARG;
    if (n_global < 0 || (n_global > 0 && !global_idx)) return SWA_ERR_ARG;
    if (!valid_scale(scale)) return SWA_ERR_ARG;
    if (!supported_d(D) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;

    std::vector<int32_t> g;
    if (n_global > 0) {
        const int st = normalize_globals(global_idx, n_global, N, g);
        if (st != SWA_OK) return st;
        if (!workspace || workspace_bytes < swa_fwd_workspace_size(B, Hq, N, D, (int)g.size()))
            return SWA_ERR_WORKSPACE;
    }

    FwdParams p;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.lse = lse;
    p.partials = (float*)workspace;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.group = Hq / Hkv;
    p.causal = win_right == 0;
    p.wl = std::min(win_left, N);   // wider windows change nothing
    p.wr = std::min(win_right, N);
    p.dil = dilation;
    p.scale_log2 = scale * kLog2e;
    swa::FwdShape shape;
    if (!plan_band(p, dtype, &shape)) return SWA_ERR_ARG;

    p.n_global = (int)g.size();
    for (int i = 0; i < p.n_global; i++) p.gpos[i] = g[i];
    global_chunks(N, &p.g_chunk, &p.g_nchunks);
    p.g_rowgroups = (int)cdiv(p.n_global, shape.grows_rows);

    hipError_t e = dtype == SWA_BF16 ? swa::launch_fwd_bf16(p, D, stream)
                                     : swa::launch_fwd_f32(p, D, stream);
    if (e != hipSuccess) return SWA_ERR_HIP;
    if (p.n_global > 0) {
        CombineParams c;
        std::memset(&c, 0, sizeof c);
        c.partials = p.partials;
        c.out = out;
        c.lse = lse;
        c.rows = B * Hq * p.n_global;
        c.splits = p.g_nchunks;
        c.mode = 1;
        c.B = B;
        c.Hq = Hq;
        c.N = N;
        c.n_global = p.n_global;
        std::memcpy(c.gpos, p.gpos, sizeof c.gpos);
        if (swa::launch_combine(c, D, dtype, stream) != hipSuccess) return SWA_ERR_HIP;
    }
    return SWA_OK;
}

int swa_kv_append(void* kcache, void* vcache, const void* k_new, const void* v_new,
                  int32_t* ring_head, int32_t* cache_len, int B, int Hkv, int W, int D,
                  int dtype, hipStream_t stream) {
    if (!kcache || !vcache || !k_new || !v_new || !ring_head || !cache_len) return SWA_ERR_ARG;
    if (B <= 0 || Hkv <= 0 || W <= 0 || D <= 0) return SWA_ERR_ARG;
    if (!supported_d(D) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
    const int elem = dtype == SWA_BF16 ? 2 : 4;
    hipError_t e = swa::launch_kv_append(kcache, vcache, k_new, v_new, ring_head, cache_len, B,
                                         Hkv, W, D, elem, stream);
    return e == hipSuccess ? SWA_OK : SWA_ERR_HIP;
}

int swa_kv_append_chunk(void* kcache, void* vcache, const void* k, const void* v,
                        int32_t* ring_head, int32_t* cache_len, int B, int Hkv, int W, int n,
                        int D, int dtype, hipStream_t stream) {
    if (!kcache || !vcache || !ring_head || !cache_len) return SWA_ERR_ARG;
    if (n > 0 && (!k || !v)) return SWA_ERR_ARG;  // an empty chunk may have no storage
    if (B <= 0 || Hkv <= 0 || W <= 0 || W > kMaxN || n < 0 || n > kMaxN || D <= 0)
        return SWA_ERR_ARG;
    if (!supported_d(D) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
    if (n == 0) return SWA_OK;
    const int elem = dtype == SWA_BF16 ? 2 : 4;
    hipError_t e = swa::launch_kv_append_chunk(kcache, vcache, k, v, ring_head, cache_len, B, Hkv,
                                               W, n, D, elem, stream);
    return e == hipSuccess ? SWA_OK : SWA_ERR_HIP;
}

int swa_fwd_cached(const void* q, const void* k, const void* v, const void* kcache,
                   const void* vcache, const int32_t* ring_head, const int32_t* cache_len,
                   void* out, float* lse, int B, int Hq, int Hkv, int n, int W, int D,
                   int win_left, float scale, int dtype, hipStream_t stream) {
    if (!q || !k || !v || !kcache || !vcache || !ring_head || !cache_len || !out)
        return SWA_ERR_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || n <= 0 || n > kMaxN || W <= 0 || W > kMaxN || D <= 0)
        return SWA_ERR_ARG;
    if (Hq % Hkv != 0 || win_left < 0 || win_left > W) return SWA_ERR_ARG;
    if (!valid_scale(scale)) return SWA_ERR_ARG;
    if (!supported_d(D) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;

    FwdParams p;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = n;
    p.group = Hq / Hkv;
    p.causal = 1;
    p.wl = win_left;   // may exceed n: the ring supplies the older keys
    p.wr = 0;
    p.dil = 1;
    p.scale_log2 = scale * kLog2e;
    p.kring = kcache;
    p.vring = vcache;
    p.ring_head = ring_head;
    p.cache_len = cache_len;
    p.W = W;
    swa::FwdShape shape;
    if (!plan_band(p, dtype, &shape)) return SWA_ERR_ARG;
    hipError_t e = dtype == SWA_BF16 ? swa::launch_fwd_bf16(p, D, stream)
                                     : swa::launch_fwd_f32(p, D, stream);
    return e == hipSuccess ? SWA_OK : SWA_ERR_HIP;
}

size_t swa_decode_sinks_workspace_size(int B, int Hq, int W, int D, int n_sink) {
    if (B <= 0 || Hq <= 0 || W <= 0 || !supported_d(D) || n_sink < 0) return 0;
    return (size_t)B * Hq * decode_max_splits(B, Hq, W, n_sink) * swa::partial_floats(D) *
           sizeof(float);
}

size_t swa_decode_workspace_size(int B, int Hq, int W, int D) {
    return swa_decode_sinks_workspace_size(B, Hq, W, D, 0);
}

int swa_decode_sinks(const void* q, const void* kcache, const void* vcache,
                     const int32_t* ring_head, const int32_t* cache_len, const void* ksink,
                     const void* vsink, int n_sink, void* out, float* lse, int B, int Hq,
                     int Hkv, int W, int D, float scale, void* workspace,
                     size_t workspace_bytes, int dtype, hipStream_t stream) {
    DecodeParams p;
    const int st = plan_ring_decode(p, q, kcache, vcache, ring_head, cache_len, ksink, vsink,
                                    n_sink, out, B, Hq, Hkv, W, D, scale, dtype);
    if (st != SWA_OK) return st;
    if (!workspace || workspace_bytes < swa_decode_sinks_workspace_size(B, Hq, W, D, n_sink))
        return SWA_ERR_WORKSPACE;
    p.partials = (float*)workspace;
    return run_decode(p, out, lse, D, dtype, false, stream);
}

int swa_decode(const void* q, const void* kcache, const void* vcache, const int32_t* ring_head,
               const int32_t* cache_len, void* out, float* lse, int B, int Hq, int Hkv, int W,
               int D, float scale, void* workspace, size_t workspace_bytes, int dtype,
               hipStream_t stream) {
    return swa_decode_sinks(q, kcache, vcache, ring_head, cache_len, nullptr, nullptr, 0, out,
                            lse, B, Hq, Hkv, W, D, scale, workspace, workspace_bytes, dtype,
                            stream);
}

int swa_kv_append_paged(void* kpool, void* vpool, const void* k, const void* v,
                        const int32_t* block_table, int32_t* seq_len, int B, int Hkv,
                        int n_pages, int page_size, int nb, int W, int n, int D, int dtype,
                        hipStream_t stream) {
    if (!kpool || !vpool || !block_table || !seq_len) return SWA_ERR_ARG;
    if (n > 0 && (!k || !v)) return SWA_ERR_ARG;
    if (B <= 0 || Hkv <= 0 || n_pages <= 0 || nb <= 0 || W <= 0 || W > kMaxN || n < 0 ||
        n > kMaxN || D <= 0)
        return SWA_ERR_ARG;
    const int sh = page_shift_of(page_size);
    if (sh < 0 || (int64_t)nb * page_size < (int64_t)W + page_size - 1) return SWA_ERR_ARG;
    if (!supported_d(D) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
    if (n == 0) return SWA_OK;
    const int elem = dtype == SWA_BF16 ? 2 : 4;
    hipError_t e = swa::launch_kv_append_paged(kpool, vpool, k, v, block_table, seq_len, B, Hkv,
                                               n_pages, sh, nb, W, n, D, elem, stream);
    return e == hipSuccess ? SWA_OK : SWA_ERR_HIP;
}

int swa_decode_paged(const void* q, const void* kpool, const void* vpool,
                     const int32_t* block_table, const int32_t* seq_len, void* out, float* lse,
                     int B, int Hq, int Hkv, int n_pages, int page_size, int nb, int W, int D,
                     float scale, void* workspace, size_t workspace_bytes, int dtype,
                     hipStream_t stream) {
    if (!q || !kpool || !vpool || !block_table || !seq_len || !out) return SWA_ERR_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || n_pages <= 0 || nb <= 0 || W <= 0 ||
        W > kMaxN || D <= 0)
        return SWA_ERR_ARG;
    const int sh = page_shift_of(page_size);
    if (sh < 0 || (int64_t)nb * page_size < (int64_t)W + page_size - 1) return SWA_ERR_ARG;
    if (!valid_scale(scale)) return SWA_ERR_ARG;
    if (!supported_d(D) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < swa_decode_workspace_size(B, Hq, W, D))
        return SWA_ERR_WORKSPACE;
    DecodeParams p;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.kcache = kpool;
    p.vcache = vpool;
    p.partials = (float*)workspace;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.W = W;
    p.group = Hq / Hkv;
    p.scale_log2 = scale * kLog2e;
    decode_splits(dtype, B, Hq, Hkv, W, &p.ring_splits, &p.slots_per_split);
    p.block_table = block_table;
    p.seq_len = seq_len;
    p.n_pages = n_pages;
    p.page_shift = sh;
    p.nb = nb;
    return run_decode(p, out, lse, D, dtype, true, stream);
}

// Workspace of swa_bwd: per-row dout . out, then (global tokens only) the
// float32 partial sums of the global rows' dq (one per key chunk) and of the
// global keys' dk, dv (one per row chunk).
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static size_t bwd_delta_bytes(int B, int Hq, int N) {
    return align256((size_t)B * Hq * N * sizeof(float));
}

// Splits of the N keys (or rows) of the global tokens' passes: about 512
// workgroups per pass for a 16-token block, each split a multiple of 32 keys.
// Independent of the number of global tokens, so that the workspace grows
// with it.
static void bwd_global_chunks(int B, int H, int N, int* chunk, int* nchunks) {
    const int64_t nc = std::min<int64_t>(cdiv(N, 256), std::max<int64_t>(1, cdiv(512, (int64_t)B * H)));
    *chunk = (int)(cdiv(cdiv(N, nc), 32) * 32);
    *nchunks = (int)cdiv(N, *chunk);
}
static size_t bwd_dq_part_bytes(int B, int Hq, int N, int ng, int D) {
    int ck, nc;
    bwd_global_chunks(B, Hq, N, &ck, &nc);
    return align256((size_t)B * Hq * ng * nc * D * sizeof(float));
}
static size_t bwd_dkv_part_bytes(int B, int Hkv, int N, int ng, int D) {
    int ck, nc;
    bwd_global_chunks(B, Hkv, N, &ck, &nc);
    return align256((size_t)B * Hkv * ng * nc * 2 * D * sizeof(float));
}

size_t swa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int D, int n_global) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || N > kMaxN || !supported_d(D)) return 0;
    if (n_global < 0) return 0;
    const int ng = std::min(n_global, std::min(N, SWA_MAX_GLOBAL));
    size_t bytes = bwd_delta_bytes(B, Hq, N);
    if (ng > 0) bytes += bwd_dq_part_bytes(B, Hq, N, ng, D) + bwd_dkv_part_bytes(B, Hkv, N, ng, D);
    return bytes;
}

int swa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int D,
            int win_left, int win_right, int dilation, const int32_t* global_idx, int n_global,
            float scale, int dtype, void* workspace, size_t workspace_bytes,
            hipStream_t stream) {
    if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return SWA_ERR_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || N > kMaxN || D <= 0) return SWA_ERR_ARG;
    if (Hq % Hkv != 0) return SWA_ERR_ARG;
    if (win_left < 0 || win_right < 0 || dilation < 1) return SWA_ERR_ARG;
    if (n_global < 0 || (n_global > 0 && !global_idx)) return SWA_ERR_ARG;
    if (!valid_scale(scale)) return SWA_ERR_ARG;
    if (!supported_d(D) || !known_dtype(dtype)) return SWA_ERR_UNSUPPORTED;
    std::vector<int32_t> g;
    if (n_global > 0) {
        const int st = normalize_globals(global_idx, n_global, N, g);
        if (st != SWA_OK) return st;
    }
    const int ng = (int)g.size();
    if (!workspace || workspace_bytes < swa_bwd_workspace_size(B, Hq, Hkv, N, D, ng))
        return SWA_ERR_WORKSPACE;

    swa::BwdParams bp;
    std::memset(&bp, 0, sizeof bp);
    FwdParams& p = bp.f;
    p.q = q;
    p.k = k;
    p.v = v;
    p.lse = const_cast<float*>(lse);
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.group = Hq / Hkv;
    p.causal = win_right == 0;
    p.wl = std::min(win_left, N);
    p.wr = std::min(win_right, N);
    p.dil = dilation;
    p.scale_log2 = scale * kLog2e;
    const swa::FwdShape shape =
        dtype == SWA_BF16 ? swa::bwd_bf16_dq_shape(p.group) : swa::bwd_f32_dq_shape(p.group);
    if (!plan_band_shape(p, shape)) return SWA_ERR_ARG;
    bp.out = out;
    bp.dout = dout;
    bp.delta = (float*)workspace;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.scale = scale;
    bp.bmk = dtype == SWA_BF16 ? swa::bwd_bf16_dkdv_keys() : swa::bwd_f32_dkdv_keys();
    bp.ktiles_long = (int)cdiv(p.qd + 1, bp.bmk);
    bp.ktiles_short = (int)cdiv(p.qd, bp.bmk);
    const int64_t per_slab =
        (int64_t)p.rem * bp.ktiles_long + (int64_t)(dilation - p.rem) * bp.ktiles_short;
    const int64_t kblocks = (int64_t)B * Hkv * per_slab;
    if (per_slab > INT32_MAX || kblocks > INT32_MAX) return SWA_ERR_ARG;
    bp.ktiles_per_slab = (int)per_slab;
    bp.k_blocks = (int)kblocks;

    // the global tokens' pairs outside the band: workgroup splits
    swa::GlobalBwdParams gb;
    std::memset(&gb, 0, sizeof gb);
    if (ng > 0) {
        gb.q = q;
        gb.k = k;
        gb.v = v;
        gb.dout = dout;
        gb.lse = lse;
        gb.delta = bp.delta;
        gb.dq = dq;
        gb.dk = dk;
        gb.dv = dv;
        char* ws = (char*)workspace + bwd_delta_bytes(B, Hq, N);
        gb.dq_part = (float*)ws;
        gb.dkv_part = (float*)(ws + bwd_dq_part_bytes(B, Hq, N, ng, D));
        gb.B = B;
        gb.Hq = Hq;
        gb.Hkv = Hkv;
        gb.N = N;
        gb.group = p.group;
        gb.wl = p.wl;
        gb.wr = p.wr;
        gb.dil = dilation;
        gb.causal = p.causal;
        gb.scale = scale;
        gb.scale_log2 = p.scale_log2;
        gb.n_global = ng;
        for (int i = 0; i < ng; i++) gb.gpos[i] = g[i];
        gb.row_tiles = gb.key_tiles = (int)cdiv(ng, swa::kGlobalBwdItems);
        // splits of the N keys (rows): each split leaves a float32 partial
        // that the add kernels sum in split order
        bwd_global_chunks(B, Hq, N, &gb.key_chunk, &gb.n_key_chunks);
        bwd_global_chunks(B, Hkv, N, &gb.row_chunk, &gb.n_row_chunks);
        gb.n_row_tiles_all = gb.n_key_tiles_all = (int)cdiv(N, 64);
        if (dtype == SWA_BF16) {
            // the bf16 dq pass walks the global keys after the band (gathered
            // tiles), which covers the pairs of the other rows with them
            p.n_global = ng;
            for (int i = 0; i < ng; i++) p.gpos[i] = g[i];
            gb.fused |= swa::kGlobalColsDqFused;
            // at D = 64 the dk/dv pass stages the global rows after the band
            // (gathered steps), which covers their pairs with every key
            if (D == 64) gb.fused |= swa::kGlobalRowsDkdvFused;
        }
        if ((int64_t)B * Hq * gb.n_row_tiles_all > INT32_MAX ||
            (int64_t)B * Hq * gb.row_tiles * gb.n_key_chunks > INT32_MAX ||
            (int64_t)B * Hkv * gb.key_tiles * gb.n_row_chunks > INT32_MAX)
            return SWA_ERR_ARG;
    }

    // (bf16: the dq pass computes each row's delta and writes it before the
    // passes that read it)
    if (dtype == SWA_F32 && swa::launch_bwd_delta(bp, D, stream) != hipSuccess)
        return SWA_ERR_HIP;
    hipError_t e = dtype == SWA_BF16 ? swa::launch_bwd_bf16(bp, D, stream)
                                     : swa::launch_bwd_f32(bp, D, stream);
    if (e == hipSuccess && ng > 0) e = swa::launch_bwd_global(gb, D, dtype, stream);
    return e == hipSuccess ? SWA_OK : SWA_ERR_HIP;
}

}  // extern "C"

// ---- allocation-free decode ---------------------------------------------------------
// swa_decode_noalloc keeps its split partials in this file-scope device array
// instead of a caller workspace.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: the device address is looked up with
// hipGetSymbolAddress once per device, with that device current, and only
// that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[SWA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device address of the current device's scratch (looked up on the first call
// made on that device).
int scratch_address(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SWA_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return SWA_ERR_HIP;
        scratch_dev[dev] = p;
    }
    *ptr = scratch_dev[dev];
    return SWA_OK;
}

}  // namespace

extern "C" int swa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                                  const int32_t* ring_head, const int32_t* cache_len, void* out,
                                  float* lse, int B, int Hq, int Hkv, int W, int D, float scale,
                                  int dtype, hipStream_t stream) {
    DecodeParams p;
    int st = plan_ring_decode(p, q, kcache, vcache, ring_head, cache_len, nullptr, nullptr, 0,
                              out, B, Hq, Hkv, W, D, scale, dtype);
    if (st != SWA_OK) return st;
    // The partial records this launch writes: one per (sequence, query head,
    // slot range); a bf16 launch with one range per ring writes out and lse
    // directly and needs none.  Every record is written before the merge reads
    // it, so nothing has to be cleared first.
    if (!(dtype == SWA_BF16 && p.ring_splits == 1)) {
        const size_t rec = (size_t)swa::partial_floats(D) * sizeof(float);
        const size_t rows = (size_t)B * Hq;
        if (rows > SWA_NOALLOC_SCRATCH_BYTES / rec / (size_t)p.ring_splits)
            return SWA_ERR_WORKSPACE;
    }
    void* ptr = nullptr;
    st = scratch_address(&ptr);
    if (st != SWA_OK) return st;
    p.partials = (float*)ptr;
    return run_decode(p, out, lse, D, dtype, false, stream);
}
