// pa_api.hip -- the C ABI (include/pa_decode.h): host-side validation,
// planning of the split-KV partitioning, workspace management, launch and
// counters.  No C++ exception crosses the ABI and no HIP call happens before
// the arguments have been validated.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "pa_decode.h"
#include "pa_launch.h"

static_assert(PA_WORKSPACE_ZERO_BYTES == pa::kWorkspaceZeroBytes, "workspace zero region");
static_assert(PA_FUSE_MAX_GROUPS == pa::kFuseMaxGroups, "in-kernel merge groups");

namespace {

thread_local std::string t_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_err = buf;
    return code;
}

struct Counters {
    std::atomic<uint64_t> calls{0}, valu{0}, mfma{0}, split{0}, merge{0}, lean{0}, append{0}, prefill{0}, fused{0};
    std::atomic<uint64_t> last_t{0}, last_np{0}, last_variant{0}, last_schedule{0};
} g_stats;

// Timeline buffer of the partitioned MFMA decode (pa_trace_set), or null.
std::atomic<uint64_t*> g_trace{nullptr};
std::atomic<int> g_trace_wgs{0};

// Validated call geometry.
struct Geometry {
    int64_t B, Hq, Hkv, D, P, NP, max_blk;
    int qg;
    int q_dtype, kv_dtype, out_dtype;
};

inline bool float_type(int32_t dt) { return dt == PA_DTYPE_BF16 || dt == PA_DTYPE_F16 || dt == PA_DTYPE_FP32; }
inline int elem_size(int32_t dt) { return dt == PA_DTYPE_FP32 ? 4 : 2; }

struct Plan {
    int variant;        // PA_VARIANT_VALU / PA_VARIANT_MFMA
    int qw;             // query heads per workgroup
    int part_tokens;
    int n_part;
    bool split;
    size_t ws_bytes;
    size_t o_offset;    // byte offset of the partial outputs inside the workspace
    size_t lse_offset;  // byte offset of the lse array inside the workspace
    bool lean;          // balanced schedule (MFMA): shares instead of partitions
    bool n_part_fixed;  // balanced schedule: share count given by the caller
    size_t meta_offset; // balanced schedule: byte offset of the tile prefix sums
    bool fit;           // fitted partitions: size chosen on the device in [fit_lo, part_tokens]
    int fit_lo;         // fitted partitions: smallest size
    int64_t fit_grid;   // fitted partitions: workgroups partitions of part_tokens may need
    size_t fit_offset;  // fitted partitions: byte offset of the chosen size
    bool fuse;          // partitions merged in the decode kernel (no merge kernel)
};

// Fitted partitions: sizes from max(kFitMinTokens, T / kFitRange) up to the
// size T the fixed schedule would take.  Fitted partitions serve calls of
// hundreds of MB, whose best fixed sizes are 512 tokens and more; below 256
// tokens a partition's own cost (page-id fetch, LDS merge, partial write)
// outweighs the balance it buys there.
constexpr int kFitMinTokens = 256;
constexpr int kFitRange = 4;
constexpr int kFitAutoMinParts = 4;
constexpr double kFitAutoMinBytes = 192e6;

// Balanced schedule: at most this many shares (workgroups) per call, so the
// workspace size does not depend on the device it runs on.
constexpr int kLeanMaxShares = 1024;
constexpr int kLeanMaxBatch = 4096;           // prefix sums live in LDS
constexpr int kLeanMinTiles = 8;              // smallest share worth a workgroup
// Units of the balanced schedule: one static unit per workgroup plus at most
// kLeanDynPerWg dynamic units per workgroup.
constexpr int64_t kLeanMaxUnits = (int64_t)kLeanMaxShares * (1 + pa::kLeanDynPerWg);
// The automatic choice takes the balanced schedule once there are at least
// this many (sequence, query block, 16-token tile) units of capacity, i.e.
// >= 1024 tiles per workgroup at 256 workgroups.  Below it, work per
// workgroup is so short that the schedule's prologue and the segments'
// serial latency cost more than the tail the partitions leave (measured: 64
// sequences x 8 query blocks x 4096 tokens run 179 us on partitions, 198 us
// balanced).
constexpr int64_t kLeanAutoMinTiles = 262144;

constexpr size_t kAlign = 256;
constexpr int32_t kAnyFloat = 0;              // check_tensor: any of the float element types
constexpr int kMaxDevices = 64;               // CU-count cache entries
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The logit multiplier: the caller's, or for PA_SCALE_DEFAULT (a NaN) the
// method's 1/sqrt(head_dim), as the fp32 value nearest to it.
float effective_scale(float scale, int64_t head_dim) {
    return std::isnan(scale) ? (float)(1.0 / std::sqrt((double)head_dim)) : scale;
}

int check_tensor(const pa_tensor* t, const char* name, int32_t dtype, int ndim) {
    if (!t) return fail(PA_EINVAL, "%s: descriptor is NULL", name);
    if (dtype == kAnyFloat ? !float_type(t->dtype) : t->dtype != dtype)
        return fail(PA_EINVAL, "%s: dtype %d, expected %s", name, t->dtype,
                    dtype == kAnyFloat ? "bf16, fp16 or fp32" : (dtype == PA_DTYPE_INT32 ? "int32" : "bf16"));
    if (t->ndim != ndim) return fail(PA_EINVAL, "%s: ndim %d, expected %d", name, t->ndim, ndim);
    for (int i = 0; i < ndim; ++i) {
        if (t->shape[i] < 0) return fail(PA_EINVAL, "%s: negative shape[%d]", name, i);
        if (t->stride[i] < 0) return fail(PA_EINVAL, "%s: negative stride[%d]", name, i);
    }
    if (t->stride[ndim - 1] != 1 && t->shape[ndim - 1] > 1)
        return fail(PA_EINVAL, "%s: innermost stride must be 1", name);
    bool empty = false;
    for (int i = 0; i < ndim; ++i) empty = empty || t->shape[i] == 0;
    if (!t->data && !empty) return fail(PA_EINVAL, "%s: data pointer is NULL", name);
    return PA_OK;
}

int check_rows16(const pa_tensor* t, const char* name, int n_outer) {
    if (!t->data) return PA_OK;   // empty tensor (checked by check_tensor)
    if (!aligned16(t->data)) return fail(PA_EALIGN, "%s: base pointer not 16-byte aligned", name);
    const int per16 = 16 / elem_size(t->dtype);   // elements per 16 bytes
    for (int i = 0; i < n_outer; ++i)
        if (t->shape[i] > 1 && (t->stride[i] % per16) != 0)
            return fail(PA_EALIGN, "%s: stride[%d]=%lld is not a multiple of %d elements (16 bytes)", name, i,
                        (long long)t->stride[i], per16);
    return PA_OK;
}

int validate(const pa_tensor* q, const pa_tensor* k, const pa_tensor* v, const pa_tensor* bt,
             const pa_tensor* ctx, float scale, int num_q_heads, int num_kv_heads, int head_dim,
             int page_size, const pa_tensor* out, const pa_opts* opts, Geometry& geo) {
    int rc;
    if ((rc = check_tensor(q, "q", kAnyFloat, 3))) return rc;
    if ((rc = check_tensor(k, "k_cache", kAnyFloat, 4))) return rc;
    if ((rc = check_tensor(v, "v_cache", kAnyFloat, 4))) return rc;
    if ((rc = check_tensor(bt, "block_tables", PA_DTYPE_INT32, 2))) return rc;
    if ((rc = check_tensor(ctx, "context_lens", PA_DTYPE_INT32, 1))) return rc;
    if ((rc = check_tensor(out, "out", kAnyFloat, 3))) return rc;
    if (k->dtype != v->dtype) return fail(PA_EINVAL, "k_cache and v_cache element types differ");
    if (std::isinf(scale)) return fail(PA_EINVAL, "scale is infinite");
    if (page_size < 1) return fail(PA_EINVAL, "page_size %d < 1", page_size);
    if (num_q_heads < 1 || num_kv_heads < 1) return fail(PA_EINVAL, "head counts must be >= 1");
    if (num_q_heads % num_kv_heads) return fail(PA_EINVAL, "num_q_heads %d not a multiple of num_kv_heads %d",
                                                num_q_heads, num_kv_heads);
    const int64_t B = q->shape[0];
    if (q->shape[1] != num_q_heads || q->shape[2] != head_dim)
        return fail(PA_EINVAL, "q shape [%lld,%lld,%lld] does not match Hq=%d, D=%d", (long long)B,
                    (long long)q->shape[1], (long long)q->shape[2], num_q_heads, head_dim);
    for (int i = 0; i < 4; ++i)
        if (k->shape[i] != v->shape[i]) return fail(PA_EINVAL, "k_cache and v_cache shapes differ");
    if (k->shape[1] != page_size || k->shape[2] != num_kv_heads || k->shape[3] != head_dim)
        return fail(PA_EINVAL, "k_cache shape [%lld,%lld,%lld,%lld] does not match P=%d, Hkv=%d, D=%d",
                    (long long)k->shape[0], (long long)k->shape[1], (long long)k->shape[2],
                    (long long)k->shape[3], page_size, num_kv_heads, head_dim);
    if (bt->shape[0] != B) return fail(PA_EINVAL, "block_tables has %lld rows, batch is %lld",
                                       (long long)bt->shape[0], (long long)B);
    if (ctx->shape[0] != B) return fail(PA_EINVAL, "context_lens has %lld entries, batch is %lld",
                                        (long long)ctx->shape[0], (long long)B);
    if (out->shape[0] != B || out->shape[1] != num_q_heads || out->shape[2] != head_dim)
        return fail(PA_EINVAL, "out shape does not match q");
    if (opts) {
        for (int i = 0; i < 2; ++i)
            if (opts->reserved[i]) return fail(PA_EINVAL, "pa_opts.reserved must be zero");
        if (opts->merge < PA_MERGE_AUTO || opts->merge > PA_MERGE_FUSED)
            return fail(PA_EINVAL, "unknown merge %d", opts->merge);
        if (opts->variant < PA_VARIANT_AUTO || opts->variant > PA_VARIANT_MFMA)
            return fail(PA_EINVAL, "unknown variant %d", opts->variant);
        if (opts->partition_tokens < 0) return fail(PA_EINVAL, "partition_tokens < 0");
        if (opts->schedule == PA_SCHEDULE_STAGED)
            return fail(PA_ENOTSUP, "the staged schedule is for several queries per sequence (pa_prefill)");
        if (opts->schedule < PA_SCHEDULE_AUTO || opts->schedule > PA_SCHEDULE_FITTED)
            return fail(PA_EINVAL, "unknown schedule %d", opts->schedule);
        if (opts->shares < 0 || opts->shares > kLeanMaxShares)
            return fail(PA_EINVAL, "shares %d outside 0..%d", opts->shares, kLeanMaxShares);
        if (opts->window < 0) return fail(PA_EINVAL, "window %d < 0", opts->window);
    }
    if (head_dim != 128 && head_dim != 256 && head_dim != 512)
        return fail(PA_ENOTSUP, "head_dim %d (supported: 128, 256, 512)", head_dim);
    const int qg = num_q_heads / num_kv_heads;
    if (qg != 1 && qg != 2 && qg != 4 && qg != 8 && qg != 16)
        return fail(PA_ENOTSUP, "Hq/Hkv = %d (supported: 1, 2, 4, 8, 16)", qg);
    if (B > 65535) return fail(PA_ENOTSUP, "batch %lld > 65535", (long long)B);
    if (bt->shape[1] > (int64_t)1 << 24 || (int64_t)bt->shape[1] * page_size > INT32_MAX / 2)
        return fail(PA_ENOTSUP, "block table too wide");
    if (k->shape[0] > INT32_MAX) return fail(PA_ENOTSUP, "pool too large");
    if ((rc = check_rows16(q, "q", 2))) return rc;
    if ((rc = check_rows16(k, "k_cache", 3))) return rc;
    if ((rc = check_rows16(v, "v_cache", 3))) return rc;
    if ((rc = check_rows16(out, "out", 2))) return rc;
    if ((reinterpret_cast<uintptr_t>(bt->data) & 3u) || (reinterpret_cast<uintptr_t>(ctx->data) & 3u))
        return fail(PA_EALIGN, "block_tables/context_lens not 4-byte aligned");
    geo = Geometry{B, num_q_heads, num_kv_heads, head_dim, page_size, k->shape[0], bt->shape[1], qg,
                   q->dtype, k->dtype, out->dtype};
    return PA_OK;
}

// Whether a call may take fitted partitions: the MFMA kernel, no window,
// lengths few enough for every workgroup to read, block tables of fewer than
// 2^24 tokens (the kernel's float-estimated divisions are exact below that),
// and no partition size given by the caller.
bool fit_allowed(const Geometry& g, const Plan& pl, const pa_opts* opts) {
    return pl.variant == PA_VARIANT_MFMA && g.B <= pa::kFitMaxBatch && g.max_blk * g.P < pa::kFitMaxTokens &&
           !(opts && opts->window > 0) && !(opts && opts->partition_tokens > 0);
}

// The automatic schedule takes fitted partitions where it would split them
// and a smaller size than the fixed one is allowed.
constexpr bool kFitAuto = true;

// Whether a split call's partitions may be merged inside the decode kernel:
// the matrix-core partition kernel (fixed or fitted), and few enough
// (sequence, query block) groups for the workspace's counters.
bool fuse_allowed(const Geometry& g, const Plan& pl) {
    return pl.variant == PA_VARIANT_MFMA && !pl.lean && g.B * (g.Hq / pl.qw) <= pa::kFuseMaxGroups;
}

// The automatic choice of the in-kernel merge: fixed partitions, at most
// two per group, and a grid of at most one workgroup per compute unit of the
// MI355X (256).  Each partition of a merged group waits for its partial
// stores to be written through before it counts itself in, and the last one
// then reads the others' partials: a serial tail of about three memory round
// trips.  That beats the merge kernel's launch and round trip only where the
// tail merges two partials and no workgroup waits for a compute unit behind
// one that is waiting (measured, per call in graphs of 64: batch16 (two
// partitions, 256 workgroups) 17.8 -> 17.0 us warm, 18.8 -> 18.2 us cold;
// slower elsewhere: single_seq (nine) 8.2 -> 8.6, hd256_gqa4 fitted 33.8 ->
// 35.1, hd512_gqa4 fitted 37.2 -> 47.6, the 4096-token window on the
// long-context batch (two partitions, 1024 workgroups) 177 -> 183).
constexpr int64_t kFuseAutoMaxWorkgroups = 256;
bool fuse_auto(const Geometry& g, const Plan& pl) {
    const int64_t groups = g.B * (g.Hq / pl.qw);
    return !pl.fit && pl.n_part <= 2 && groups * pl.n_part <= kFuseAutoMaxWorkgroups;
}

Plan make_plan(const Geometry& g, const pa_opts* opts) {
    Plan pl{};
    const int qw_mfma = g.qg < 16 ? g.qg : 16;
    if (opts && opts->variant)
        pl.variant = opts->variant;
    else
        pl.variant = pa::mfma_supported((int)g.D, qw_mfma, g.kv_dtype) ? PA_VARIANT_MFMA : PA_VARIANT_VALU;
    if (pl.variant == PA_VARIANT_MFMA)
        pl.qw = qw_mfma;                        // one 16-column MFMA tile of queries
    else
        pl.qw = std::min(g.qg, g.D == 512 ? 2 : 8);   // query rows that fit the VALU registers
    // Tokens a sequence's work can span: the block table's capacity, or with
    // a window of W the W tokens plus up to 15 before them (work starts on a
    // 16-token tile boundary).
    int64_t max_ctx = std::max<int64_t>(g.max_blk * g.P, 1);
    if (opts && opts->window > 0) max_ctx = std::min<int64_t>(max_ctx, (int64_t)opts->window + 15);
    const int64_t groups = g.B * (g.Hq / pl.qw);

    // Balanced schedule (MFMA): equal shares of all (sequence, query block,
    // tile) work, whatever the mix of sequence lengths.
    const int64_t ub_tiles = groups * ((max_ctx + 15) / 16);
    const int sched = opts ? opts->schedule : PA_SCHEDULE_AUTO;
    const bool lean_ok = pl.variant == PA_VARIANT_MFMA && pa::mfma_lean_supported((int)g.D, pl.qw, g.kv_dtype) &&
                         g.B <= kLeanMaxBatch && ub_tiles < ((int64_t)1 << 30);
    if (sched == PA_SCHEDULE_BALANCED)
        pl.lean = lean_ok;
    else if (sched == PA_SCHEDULE_AUTO)
        pl.lean = lean_ok && !(opts && opts->partition_tokens > 0) && ub_tiles >= kLeanAutoMinTiles;
    else
        pl.lean = false;
    if (pl.lean) {
        const int64_t n_wg = std::max<int64_t>(1, std::min<int64_t>(kLeanMaxShares, ub_tiles / kLeanMinTiles));
        pl.n_part_fixed = opts && opts->shares > 0;
        pl.n_part = pl.n_part_fixed ? opts->shares : (int)n_wg;   // shares (workgroups)
        pl.part_tokens = 0;
        pl.split = true;
        // One partial slot row per (group, unit) piece: groups + units at most.
        const size_t slots = (size_t)(groups + kLeanMaxUnits) * pl.qw;
        pl.o_offset = pa::kWorkspaceZeroBytes;
        pl.lse_offset = pl.o_offset + align_up(slots * g.D * sizeof(float), kAlign);
        pl.meta_offset = pl.lse_offset + align_up(slots * sizeof(float), kAlign);
        pl.ws_bytes = pl.meta_offset + align_up((size_t)(g.B + 4) * sizeof(int), kAlign);
        return pl;
    }

    int64_t T;
    if (opts && opts->partition_tokens > 0) {
        T = (int64_t)opts->partition_tokens;
    } else if (pl.variant == PA_VARIANT_MFMA) {
        // Few, long partitions: each workgroup's fixed cost (page-table
        // fetch, LDS merge, partial write) is paid per partition, so aim for
        // about one workgroup per CU of work, partitions of 64..4096 tokens
        // (measured per call: one 1152-token sequence, 8 KV heads, runs 7.7 us
        // at 64, 8.6 at 128; four of them 10.5 at 128, 9.9 at 192, 11.0 at
        // 256; one 4096-token sequence 14.4 at 64, 11.0 at 128, 11.4 at 256).
        // Partitions of 64 tokens only where they give at least four per
        // table: a call that would split into two or three (the tiny
        // batch: 5.1 us unsplit at 128, 6.4 us at 64) stays at 128.
        T = (max_ctx * groups + 255) / 256;
        T = std::max<int64_t>(64, std::min<int64_t>(T, 4096));
        if (T <= 64 && (max_ctx + 63) / 64 < 4) T = 128;
    } else {
        // Aim for ~1024 workgroups; partitions of 64..1024 tokens.
        T = (max_ctx * groups + 1023) / 1024;
        T = std::max<int64_t>(64, std::min<int64_t>(T, 1024));
    }
    T = (T + 63) / 64 * 64;
    // Page-id LDS stays <= ~32 KB (16 KB beside the d512 MFMA merge buffer,
    // 130 KB, inside the CU's 160 KB).
    const bool big_merge = pl.variant == PA_VARIANT_MFMA && g.D == 512;
    T = std::min<int64_t>(T, (big_merge ? 4096 : 8192) * g.P);
    if (T >= max_ctx) T = max_ctx;
    pl.part_tokens = (int)T;
    pl.n_part = (int)((max_ctx + T - 1) / T);
    pl.split = pl.n_part > 1;
    // Fitted partitions: the device picks the size in [fit_lo, T] from the
    // actual lengths; the partial slots cover the smallest size.
    pl.fit = pl.split && (sched == PA_SCHEDULE_FITTED || (sched == PA_SCHEDULE_AUTO && kFitAuto)) &&
             fit_allowed(g, pl, opts);
    if (pl.fit) {
        pl.fit_lo = (int)std::min<int64_t>(T, (std::max<int64_t>(kFitMinTokens, T / kFitRange) + 63) / 64 * 64);
        // The automatic choice keeps fixed partitions when there is no
        // smaller size to pick, or when the block table holds fewer than
        // kFitAutoMinParts fixed partitions: the fitted prologue (the
        // lengths read first, the size search) costs about 1 us, which pays
        // only where sequences much shorter than the table leave compute
        // units idle (measured: 32 sequences of 512..4096 tokens in a
        // 4096-token table, decode kernel 31.7 -> 29.0 us; 16 sequences of
        // 1024..1152 tokens in a 1152-token table, 14.4 -> 15.4 us).
        // The gain grows with the call, the cost does not: the KV the
        // block tables can hold must also take at least ~24 us at HBM peak
        // (measured: the same batch at half the lengths, 2048-token tables,
        // ran 20.6 us on fixed and 21.3 us on fitted partitions).
        const double cap_bytes = (double)g.B * (double)max_ctx * (double)g.Hkv * (double)g.D * 2.0 *
                                 (double)elem_size(g.kv_dtype);
        if (sched == PA_SCHEDULE_AUTO &&
            (pl.fit_lo == T || pl.n_part < kFitAutoMinParts || cap_bytes < kFitAutoMinBytes))
            pl.fit = false;
    }
    if (pl.fit) {
        pl.fit_grid = (int64_t)pl.n_part * groups;
        pl.n_part = (int)((max_ctx + pl.fit_lo - 1) / pl.fit_lo);
    }
    // Partitions merged inside the decode kernel: the matrix-core partition
    // kernel only, one arrival counter per group in the workspace's zero
    // region.
    const int merge = opts ? opts->merge : PA_MERGE_AUTO;
    pl.fuse = pl.split && merge != PA_MERGE_KERNEL && fuse_allowed(g, pl) &&
              (merge == PA_MERGE_FUSED || fuse_auto(g, pl));
    if (pl.split) {
        // The counters keep their place at the start, so one workspace can
        // serve every schedule.
        const size_t n = (size_t)g.B * g.Hq * pl.n_part;
        pl.o_offset = pa::kWorkspaceZeroBytes;
        pl.lse_offset = pl.o_offset + align_up(n * g.D * sizeof(float), kAlign);
        pl.ws_bytes = pl.lse_offset + align_up(n * sizeof(float), kAlign);
        if (pl.fit) {
            // the size picked, then one hint (the triple taken by the same
            // workgroup in the previous call) per workgroup the grid can have
            pl.fit_offset = pl.ws_bytes;
            pl.ws_bytes += kAlign + align_up((size_t)std::max<int64_t>(pl.fit_grid, kLeanMaxShares) * 16, kAlign);
        }
    }
    return pl;
}

// Library-owned per-device workspace.  A buffer that is outgrown is kept,
// not freed, until pa_release: work enqueued earlier may still use it, and
// freeing it here would need a device-wide synchronisation.
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    std::vector<void*> retired;
};
std::mutex g_ws_mu;
std::vector<Workspace> g_ws;

int library_workspace(int dev, size_t need, hipStream_t stream, void** out) {
    // A captured call would bake the library's buffer into the graph; the
    // buffer can be outgrown (and released) by later calls, so captured calls
    // must bring their own workspace (pa_decode_ex, pa_prefill) or use the
    // static one of pa_decode_noalloc.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return fail(PA_EHIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
    if (cs != hipStreamCaptureStatusNone)
        return fail(PA_EINVAL, "the stream is being captured: the library's own workspace cannot be used in a "
                               "graph; pass a workspace (pa_decode_ex / pa_prefill) or call pa_decode_noalloc");
    std::lock_guard<std::mutex> lk(g_ws_mu);
    if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
    Workspace& w = g_ws[dev];
    if (w.bytes < need) {
        const size_t sz = align_up(need + need / 2, 1 << 20);
        void* ptr = nullptr;
        e = hipMalloc(&ptr, sz);
        if (e != hipSuccess) return fail(PA_ENOMEM, "hipMalloc(%zu): %s", sz, hipGetErrorString(e));
        // The workspace's counters must start at zero (every call leaves
        // them so); the zeroing is ordered before the call's kernels by the
        // stream.
        e = hipMemsetAsync(ptr, 0, pa::kWorkspaceZeroBytes, stream);
        if (e != hipSuccess) {
            (void)hipFree(ptr);
            return fail(PA_EHIP, "hipMemsetAsync: %s", hipGetErrorString(e));
        }
        if (w.ptr) {
            try {
                w.retired.push_back(w.ptr);
            } catch (...) {
                (void)hipFree(ptr);
                return fail(PA_ENOMEM, "host allocation failed");
            }
        }
        w.ptr = ptr;
        w.bytes = sz;
    }
    *out = w.ptr;
    return PA_OK;
}

// Compute units of a device, cached (the attribute query costs a runtime call).
int cu_count(int dev) {
    static std::atomic<int> cache[kMaxDevices];
    if (dev < 0 || dev >= kMaxDevices) return 1;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 1;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int check_plan(const Geometry& g, const Plan& pl, const pa_opts* opts) {
    if (pl.variant == PA_VARIANT_MFMA && !pa::mfma_supported((int)g.D, pl.qw, g.kv_dtype))
        return fail(PA_ENOTSUP, "MFMA variant does not support D=%lld, qg=%d, K/V dtype %d (D 128/256/512, "
                    "bf16 or fp16 K/V)", (long long)g.D, g.qg, g.kv_dtype);
    if (pl.variant == PA_VARIANT_VALU && !pa::valu_supported((int)g.D, pl.qw, g.kv_dtype))
        return fail(PA_ENOTSUP, "vector-ALU variant does not support D=%lld, qg=%d", (long long)g.D, g.qg);
    if (opts && opts->schedule == PA_SCHEDULE_BALANCED && !pl.lean)
        return fail(PA_ENOTSUP, "balanced schedule needs the MFMA variant, head_dim 128/256 and at most %d sequences",
                    kLeanMaxBatch);
    if (opts && opts->merge == PA_MERGE_FUSED && !fuse_allowed(g, pl))
        return fail(PA_ENOTSUP, "the in-kernel merge needs the MFMA partition schedules (fixed or fitted) and at "
                    "most %d (sequence, query block) groups", pa::kFuseMaxGroups);
    if (opts && opts->schedule == PA_SCHEDULE_FITTED && !fit_allowed(g, pl, opts))
        return fail(PA_ENOTSUP, "fitted partitions need the MFMA variant, no window, no partition size, at most "
                    "%d sequences and block tables of fewer than %d tokens", pa::kFitMaxBatch, pa::kFitMaxTokens);
    return PA_OK;
}

int launch(const pa_tensor* q, const pa_tensor* k, const pa_tensor* v, const pa_tensor* bt,
           const pa_tensor* ctx, float scale, const pa_tensor* out, void* stream,
           const Geometry& g, const Plan& pl, const pa_opts* opts, void* ws, int dev) {
    pa::DecodeParams p{};
    p.q = q->data;
    p.q_dtype = g.q_dtype;
    p.out_dtype = g.out_dtype;
    p.q_sb = q->stride[0];
    p.q_sh = q->stride[1];
    p.k = k->data;
    p.k_sp = k->stride[0];
    p.k_ss = k->stride[1];
    p.k_sh = k->stride[2];
    p.v = v->data;
    p.v_sp = v->stride[0];
    p.v_ss = v->stride[1];
    p.v_sh = v->stride[2];
    p.bt = static_cast<const int32_t*>(bt->data);
    p.bt_sb = bt->stride[0];
    p.ctx = static_cast<const int32_t*>(ctx->data);
    p.out = out->data;
    p.o_sb = out->stride[0];
    p.o_sh = out->stride[1];
    p.part_o = pl.split ? reinterpret_cast<float*>(static_cast<char*>(ws) + pl.o_offset) : nullptr;
    p.part_lse = pl.split ? reinterpret_cast<float*>(static_cast<char*>(ws) + pl.lse_offset) : nullptr;
    p.B = (int)g.B;
    p.Hq = (int)g.Hq;
    p.Hkv = (int)g.Hkv;
    p.P = (int)g.P;
    p.p_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((int64_t)1 << sh == g.P) p.p_shift = sh;
    p.max_blk = (int)g.max_blk;
    p.num_pages = (int)std::max<int64_t>(g.NP, 1);
    p.part_tokens = pl.part_tokens;
    p.n_part = pl.n_part;
    p.qw = pl.qw;
    p.window = opts ? opts->window : 0;
    p.scale_log2 = effective_scale(scale, g.D) * pa::kLog2e;
    hipStream_t s = static_cast<hipStream_t>(stream);

    hipError_t e;
    if (pl.lean) {
        p.lean_meta = reinterpret_cast<int*>(static_cast<char*>(ws) + pl.meta_offset);
        p.lean_ctr = static_cast<int*>(ws);
        p.lean_page_slots = pa::lean_page_slots(p.P);
        // One share per CU.  Each CU streams at a bounded rate, so the call
        // lasts as long as the most loaded CU: share counts that are not a
        // multiple of the CU count leave some CUs with one share more
        // (measured: 272 shares on 256 CUs run 1.33x longer than 256), and
        // a second share per CU brings no more bandwidth.
        const int n_wg = pl.n_part_fixed ? pl.n_part : std::min(pl.n_part, cu_count(dev));
        e = pa::launch_mfma_lean(p, (int)g.D, g.kv_dtype, n_wg, s);
        if (e != hipSuccess) return fail(PA_EHIP, "decode (mfma, balanced) launch: %s", hipGetErrorString(e));
        g_stats.mfma++;
        g_stats.lean++;
        g_stats.merge++;
        g_stats.split++;
        g_stats.calls++;
        g_stats.last_t = 0;
        g_stats.last_np = (uint64_t)n_wg;
        g_stats.last_variant = (uint64_t)pl.variant;
        g_stats.last_schedule = PA_SCHEDULE_BALANCED;
        return PA_OK;
    }
    if (pl.fit) {
        p.fit_part = reinterpret_cast<int*>(static_cast<char*>(ws) + pl.fit_offset);
        p.fit_hint = reinterpret_cast<int*>(static_cast<char*>(ws) + pl.fit_offset + kAlign);
        p.fit_lo = pl.fit_lo;
        p.fit_target = opts && opts->shares > 0 ? opts->shares : cu_count(dev);
        p.n_wg = (int)std::max<int64_t>(pl.fit_grid, p.fit_target);
    }
    if (pl.fuse) p.fuse_ctr = reinterpret_cast<int*>(static_cast<char*>(ws) + pa::kFuseCounterOffset);
    p.trace = g_trace.load();
    p.trace_wgs = p.trace ? g_trace_wgs.load() : 0;
    if (pl.variant == PA_VARIANT_MFMA) {
        e = pa::launch_mfma(p, (int)g.D, g.kv_dtype, pl.qw, pl.split, s);
        if (e != hipSuccess) return fail(PA_EHIP, "decode (mfma) launch: %s", hipGetErrorString(e));
        g_stats.mfma++;
    } else {
        e = pa::launch_valu(p, (int)g.D, g.kv_dtype, pl.qw, pl.split, s);
        if (e != hipSuccess) return fail(PA_EHIP, "decode (valu) launch: %s", hipGetErrorString(e));
        g_stats.valu++;
    }
    if (pl.split) {
        if (pl.fuse) {
            g_stats.fused++;
        } else {
            e = pa::launch_merge(p, (int)g.D, s);
            if (e != hipSuccess) return fail(PA_EHIP, "merge launch: %s", hipGetErrorString(e));
            g_stats.merge++;
        }
        g_stats.split++;
    }
    g_stats.calls++;
    g_stats.last_t = (uint64_t)pl.part_tokens;
    g_stats.last_np = (uint64_t)pl.n_part;
    g_stats.last_variant = (uint64_t)pl.variant;
    g_stats.last_schedule = pl.fit ? PA_SCHEDULE_FITTED : PA_SCHEDULE_PARTITIONS;
    return PA_OK;
}

int decode_impl(const pa_tensor* q, const pa_tensor* k, const pa_tensor* v, const pa_tensor* bt,
                const pa_tensor* ctx, float scale, int num_q_heads, int num_kv_heads, int head_dim,
                int page_size, const pa_tensor* out, void* stream, const pa_opts* opts,
                void* workspace, size_t workspace_bytes) {
    t_err.clear();
    Geometry g;
    int rc = validate(q, k, v, bt, ctx, scale, num_q_heads, num_kv_heads, head_dim, page_size, out,
                      opts, g);
    if (rc) return rc;
    Plan pl = make_plan(g, opts);
    rc = check_plan(g, pl, opts);
    if (rc) return rc;
    if (g.B == 0) return PA_OK;
    int dev = 0;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(PA_ENODEV, "no HIP device");
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ENODEV, "hipGetDevice: %s", hipGetErrorString(e));
    void* ws = nullptr;
    if (pl.split) {
        if (workspace) {
            if (workspace_bytes < pl.ws_bytes)
                return fail(PA_ENOMEM, "workspace of %zu bytes, %zu needed", workspace_bytes, pl.ws_bytes);
            if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
                return fail(PA_EALIGN, "workspace not %zu-byte aligned", kAlign);
            ws = workspace;
        } else {
            rc = library_workspace(dev, pl.ws_bytes, static_cast<hipStream_t>(stream), &ws);
            if (rc) return rc;
        }
    }
    try {
        return launch(q, k, v, bt, ctx, scale, out, stream, g, pl, opts, ws, dev);
    } catch (const std::bad_alloc&) {
        return fail(PA_ENOMEM, "host allocation failed");
    } catch (...) {
        return fail(PA_EHIP, "unexpected exception");
    }
}

// ---------------------------------------------------------------- static scratch
// The split-KV scratch of pa_decode_noalloc, for callers that cannot
// allocate: one array per device, held until the process ends.  Host code
// never uses the name `scratch` as an address (in host code it is a
// stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Zero the first n dwords (the workspace's counters).
__global__ void pa_scratch_clear_kernel(uint32_t* p, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];               // device address of `scratch` per device

int device_scratch(int dev, hipStream_t stream, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(PA_ENODEV, "device %d beyond the library's %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        // Set-up, once per device (the current one): outside stream capture,
        // since the runtime may load the module's data here.
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return fail(PA_EHIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
        if (cs != hipStreamCaptureStatusNone)
            return fail(PA_EINVAL, "the first pa_decode_noalloc call on a device sets up its scratch and must "
                                   "not be captured; make one uncaptured call first");
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(PA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        // The array starts zeroed; the counters are cleared once more here,
        // ordered before this call's kernels by the stream.
        constexpr int kWords = pa::kWorkspaceZeroBytes / (int)sizeof(uint32_t);
        hipLaunchKernelGGL(pa_scratch_clear_kernel, dim3((kWords + 255) / 256), dim3(256), 0, stream,
                           static_cast<uint32_t*>(ptr), kWords);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(PA_EHIP, "scratch clear launch: %s", hipGetErrorString(e));
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return PA_OK;
}

int decode_noalloc_impl(const pa_tensor* q, const pa_tensor* k, const pa_tensor* v, const pa_tensor* bt,
                        const pa_tensor* ctx, float scale, int num_q_heads, int num_kv_heads, int head_dim,
                        int page_size, const pa_tensor* out, void* stream, const pa_opts* opts) {
    t_err.clear();
    Geometry g;
    int rc = validate(q, k, v, bt, ctx, scale, num_q_heads, num_kv_heads, head_dim, page_size, out, opts, g);
    if (rc) return rc;
    Plan pl = make_plan(g, opts);
    rc = check_plan(g, pl, opts);
    if (rc) return rc;
    if (pl.split && pl.ws_bytes > kScratchBytes)
        return fail(PA_ENOMEM, "the call needs %zu bytes of split-KV scratch; pa_decode_noalloc has %zu "
                    "(use pa_decode_ex with a workspace)", pl.ws_bytes, kScratchBytes);
    if (g.B == 0) return PA_OK;
    int dev = 0, ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(PA_ENODEV, "no HIP device");
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ENODEV, "hipGetDevice: %s", hipGetErrorString(e));
    void* ws = nullptr;
    if (pl.split) {
        rc = device_scratch(dev, static_cast<hipStream_t>(stream), &ws);
        if (rc) return rc;
    }
    try {
        return launch(q, k, v, bt, ctx, scale, out, stream, g, pl, opts, ws, dev);
    } catch (...) {
        return fail(PA_EHIP, "unexpected exception");
    }
}

int validate_append(const pa_tensor* kn, const pa_tensor* vn, const pa_tensor* k, const pa_tensor* v,
                    const pa_tensor* bt, const pa_tensor* ctx, int num_kv_heads, int head_dim,
                    int page_size) {
    int rc;
    if ((rc = check_tensor(kn, "k_new", kAnyFloat, 3))) return rc;
    if ((rc = check_tensor(vn, "v_new", kAnyFloat, 3))) return rc;
    if ((rc = check_tensor(k, "k_cache", kAnyFloat, 4))) return rc;
    if ((rc = check_tensor(v, "v_cache", kAnyFloat, 4))) return rc;
    if (kn->dtype != k->dtype || vn->dtype != k->dtype || v->dtype != k->dtype)
        return fail(PA_EINVAL, "k_new, v_new, k_cache and v_cache must share their element type");
    if ((rc = check_tensor(bt, "block_tables", PA_DTYPE_INT32, 2))) return rc;
    if ((rc = check_tensor(ctx, "context_lens", PA_DTYPE_INT32, 1))) return rc;
    if (page_size < 1) return fail(PA_EINVAL, "page_size %d < 1", page_size);
    if (num_kv_heads < 1) return fail(PA_EINVAL, "num_kv_heads must be >= 1");
    if (head_dim < 8 || head_dim * elem_size(k->dtype) % 16)
        return fail(PA_ENOTSUP, "head_dim %d: rows are not whole 16-byte chunks", head_dim);
    const int64_t B = kn->shape[0];
    for (int i = 0; i < 3; ++i)
        if (vn->shape[i] != kn->shape[i]) return fail(PA_EINVAL, "k_new and v_new shapes differ");
    if (kn->shape[1] != num_kv_heads || kn->shape[2] != head_dim)
        return fail(PA_EINVAL, "k_new shape does not match Hkv=%d, D=%d", num_kv_heads, head_dim);
    for (int i = 0; i < 4; ++i)
        if (k->shape[i] != v->shape[i]) return fail(PA_EINVAL, "k_cache and v_cache shapes differ");
    if (k->shape[1] != page_size || k->shape[2] != num_kv_heads || k->shape[3] != head_dim)
        return fail(PA_EINVAL, "k_cache shape does not match P=%d, Hkv=%d, D=%d", page_size, num_kv_heads,
                    head_dim);
    if (bt->shape[0] != B) return fail(PA_EINVAL, "block_tables has %lld rows, batch is %lld",
                                       (long long)bt->shape[0], (long long)B);
    if (ctx->shape[0] != B) return fail(PA_EINVAL, "context_lens has %lld entries, batch is %lld",
                                        (long long)ctx->shape[0], (long long)B);
    if (B > INT32_MAX) return fail(PA_ENOTSUP, "batch too large");
    if (bt->shape[1] > (int64_t)1 << 24 || (int64_t)bt->shape[1] * page_size > INT32_MAX / 2)
        return fail(PA_ENOTSUP, "block table too wide");
    if (k->shape[0] > INT32_MAX) return fail(PA_ENOTSUP, "pool too large");
    if ((int64_t)num_kv_heads * head_dim / 8 > (1 << 20)) return fail(PA_ENOTSUP, "rows too wide");
    if ((rc = check_rows16(kn, "k_new", 2))) return rc;
    if ((rc = check_rows16(vn, "v_new", 2))) return rc;
    if ((rc = check_rows16(k, "k_cache", 3))) return rc;
    if ((rc = check_rows16(v, "v_cache", 3))) return rc;
    if ((reinterpret_cast<uintptr_t>(bt->data) & 3u) || (reinterpret_cast<uintptr_t>(ctx->data) & 3u))
        return fail(PA_EALIGN, "block_tables / context_lens not 4-byte aligned");
    if (bt->shape[0] > 1 && bt->shape[1] > 0 && bt->stride[1] != 1)
        return fail(PA_EINVAL, "block_tables: innermost stride must be 1");
    return PA_OK;
}

// ---------------------------------------------------------------- several queries
struct PrefillPlan {
    bool staged;        // eight query blocks per workgroup (no split)
    int n_slots;        // query-block slots (an upper bound on the blocks); staged: workgroup slots
    int part_tokens;
    int n_part;
    bool split;
    size_t ws_bytes, o_offset, lse_offset;
};

int validate_prefill(const pa_tensor* q, const pa_tensor* k, const pa_tensor* v, const pa_tensor* bt,
                     const pa_tensor* ctx, const pa_tensor* qs, float scale, int num_q_heads,
                     int num_kv_heads, int head_dim, int page_size, const pa_tensor* out,
                     const pa_opts* opts, Geometry& geo, int64_t& rows) {
    int rc;
    if ((rc = check_tensor(q, "q", kAnyFloat, 3))) return rc;
    if ((rc = check_tensor(k, "k_cache", kAnyFloat, 4))) return rc;
    if ((rc = check_tensor(v, "v_cache", kAnyFloat, 4))) return rc;
    if ((rc = check_tensor(bt, "block_tables", PA_DTYPE_INT32, 2))) return rc;
    if ((rc = check_tensor(ctx, "context_lens", PA_DTYPE_INT32, 1))) return rc;
    if ((rc = check_tensor(qs, "query_start", PA_DTYPE_INT32, 1))) return rc;
    if ((rc = check_tensor(out, "out", kAnyFloat, 3))) return rc;
    if (k->dtype != v->dtype) return fail(PA_EINVAL, "k_cache and v_cache element types differ");
    if (std::isinf(scale)) return fail(PA_EINVAL, "scale is infinite");
    if (page_size < 1) return fail(PA_EINVAL, "page_size %d < 1", page_size);
    if (num_q_heads < 1 || num_kv_heads < 1) return fail(PA_EINVAL, "head counts must be >= 1");
    if (num_q_heads % num_kv_heads)
        return fail(PA_EINVAL, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads, num_kv_heads);
    rows = q->shape[0];
    const int64_t B = bt->shape[0];
    if (q->shape[1] != num_q_heads || q->shape[2] != head_dim)
        return fail(PA_EINVAL, "q shape does not match Hq=%d, D=%d", num_q_heads, head_dim);
    for (int i = 0; i < 4; ++i)
        if (k->shape[i] != v->shape[i]) return fail(PA_EINVAL, "k_cache and v_cache shapes differ");
    if (k->shape[1] != page_size || k->shape[2] != num_kv_heads || k->shape[3] != head_dim)
        return fail(PA_EINVAL, "k_cache shape does not match P=%d, Hkv=%d, D=%d", page_size, num_kv_heads,
                    head_dim);
    if (ctx->shape[0] != B) return fail(PA_EINVAL, "context_lens has %lld entries, block_tables %lld rows",
                                        (long long)ctx->shape[0], (long long)B);
    if (qs->shape[0] != B + 1) return fail(PA_EINVAL, "query_start has %lld entries, %lld expected",
                                           (long long)qs->shape[0], (long long)(B + 1));
    if (out->shape[0] != rows || out->shape[1] != num_q_heads || out->shape[2] != head_dim)
        return fail(PA_EINVAL, "out shape does not match q");
    if (opts) {
        for (int i = 0; i < 2; ++i)
            if (opts->reserved[i]) return fail(PA_EINVAL, "pa_opts.reserved must be zero");
        if (opts->merge == PA_MERGE_FUSED)
            return fail(PA_ENOTSUP, "several-query attention merges split partitions in a kernel of its own");
        if (opts->merge < PA_MERGE_AUTO || opts->merge > PA_MERGE_FUSED)
            return fail(PA_EINVAL, "unknown merge %d", opts->merge);
        if (opts->variant != PA_VARIANT_AUTO && opts->variant != PA_VARIANT_MFMA)
            return fail(PA_ENOTSUP, "several-query attention runs on the MFMA kernel only");
        if (opts->partition_tokens < 0) return fail(PA_EINVAL, "partition_tokens < 0");
        if (opts->schedule == PA_SCHEDULE_BALANCED || opts->schedule == PA_SCHEDULE_FITTED)
            return fail(PA_ENOTSUP, "several-query attention uses the partition or staged schedule");
        if (opts->schedule < PA_SCHEDULE_AUTO || opts->schedule > PA_SCHEDULE_FITTED)
            return fail(PA_EINVAL, "unknown schedule %d", opts->schedule);
        if (opts->schedule == PA_SCHEDULE_STAGED && opts->partition_tokens > 0)
            return fail(PA_EINVAL, "the staged schedule has no partitions (partition_tokens must be 0)");
        if (opts->shares != 0) return fail(PA_EINVAL, "shares apply to the balanced schedule only");
        if (opts->window < 0) return fail(PA_EINVAL, "window %d < 0", opts->window);
    }
    const int qg = num_q_heads / num_kv_heads;
    if (qg != 1 && qg != 2 && qg != 4 && qg != 8 && qg != 16)
        return fail(PA_ENOTSUP, "Hq/Hkv = %d (supported: 1, 2, 4, 8, 16)", qg);
    if (!pa::prefill_supported(head_dim, k->dtype))
        return fail(PA_ENOTSUP, "several-query attention needs head_dim 128/256/512 and a bf16 or fp16 cache");
    if (B > kLeanMaxBatch) return fail(PA_ENOTSUP, "batch %lld > %d", (long long)B, kLeanMaxBatch);
    if (rows > INT32_MAX / 4) return fail(PA_ENOTSUP, "too many query rows");
    if (bt->shape[1] > (int64_t)1 << 24 || (int64_t)bt->shape[1] * page_size > INT32_MAX / 2)
        return fail(PA_ENOTSUP, "block table too wide");
    if (k->shape[0] > INT32_MAX) return fail(PA_ENOTSUP, "pool too large");
    if ((rc = check_rows16(q, "q", 2))) return rc;
    if ((rc = check_rows16(k, "k_cache", 3))) return rc;
    if ((rc = check_rows16(v, "v_cache", 3))) return rc;
    if ((rc = check_rows16(out, "out", 2))) return rc;
    if ((reinterpret_cast<uintptr_t>(bt->data) & 3u) || (reinterpret_cast<uintptr_t>(ctx->data) & 3u) ||
        (reinterpret_cast<uintptr_t>(qs->data) & 3u))
        return fail(PA_EALIGN, "block_tables / context_lens / query_start not 4-byte aligned");
    if (B > 0 && bt->shape[1] > 1 && bt->stride[1] != 1)
        return fail(PA_EINVAL, "block_tables: innermost stride must be 1");
    geo = Geometry{B, num_q_heads, num_kv_heads, head_dim, page_size, k->shape[0], bt->shape[1], qg,
                   q->dtype, k->dtype, out->dtype};
    return PA_OK;
}

// The staged kernel addresses the pool with a 32-bit page stride and a
// 24-bit slot stride (P slots of at most 2^31 elements).
bool staged_strides_ok(int64_t sp, int64_t ss, int64_t P) {
    return sp >= 0 && sp < ((int64_t)1 << 32) && ss >= 0 && ss < ((int64_t)1 << 23) && P * ss + 512 <= ((int64_t)1 << 31);
}

PrefillPlan plan_prefill(const Geometry& g, int64_t rows, const pa_opts* opts, bool staged_ok = true) {
    PrefillPlan pl{};
    const int qt = 16 / g.qg;
    const int sched = opts ? opts->schedule : PA_SCHEDULE_AUTO;
    // Staged: slots of kStagedWaves query blocks, an upper bound over any
    // split of the rows into B sequences (each sequence rounds up once).
    const int64_t gq = (int64_t)pa::kStagedWaves * qt;
    const int64_t staged_slots = (rows + gq - 1) / gq + g.B;
    if ((sched == PA_SCHEDULE_STAGED && staged_ok) ||
        (sched == PA_SCHEDULE_AUTO && staged_ok && !(opts && opts->partition_tokens > 0) && rows >= 2 * qt * g.B &&
         staged_slots * g.Hkv >= 256)) {
        pl.staged = true;
        pl.n_slots = (int)std::min<int64_t>(staged_slots, INT32_MAX);
        pl.part_tokens = 0;
        pl.n_part = 1;
        return pl;
    }
    pl.n_slots = (int)((rows + qt - 1) / qt + g.B);
    // Span of one block's work: the whole table, or with a window W the
    // block's W + qt - 1 attended tokens from a 16-token tile boundary.
    int64_t span = std::max<int64_t>(g.max_blk * g.P, 1);
    if (opts && opts->window > 0) span = std::min<int64_t>(span, (int64_t)opts->window + qt + 15);
    const int64_t blocks = (int64_t)pl.n_slots * g.Hkv;
    int64_t T;
    if (opts && opts->partition_tokens > 0) {
        T = (opts->partition_tokens + 63) / 64 * 64;
    } else if (blocks >= 256) {
        T = span;                               // enough query blocks to fill the chip: no split
    } else {
        T = (span * blocks + 255) / 256;
        T = std::max<int64_t>(256, std::min<int64_t>(T, 4096));
        T = (T + 63) / 64 * 64;
    }
    if (T >= span) T = span;
    pl.part_tokens = (int)T;
    pl.n_part = (int)((span + T - 1) / T);
    pl.split = pl.n_part > 1;
    if (pl.split) {
        const size_t n = (size_t)rows * g.Hq * pl.n_part;
        pl.o_offset = pa::kWorkspaceZeroBytes;
        pl.lse_offset = pl.o_offset + align_up(n * g.D * sizeof(float), kAlign);
        pl.ws_bytes = pl.lse_offset + align_up(n * sizeof(float), kAlign);
    }
    return pl;
}

int prefill_impl(const pa_tensor* q, const pa_tensor* k, const pa_tensor* v, const pa_tensor* bt,
                 const pa_tensor* ctx, const pa_tensor* qs, float scale, int num_q_heads, int num_kv_heads,
                 int head_dim, int page_size, const pa_tensor* out, void* stream, const pa_opts* opts,
                 void* workspace, size_t workspace_bytes) {
    t_err.clear();
    Geometry g;
    int64_t rows = 0;
    int rc = validate_prefill(q, k, v, bt, ctx, qs, scale, num_q_heads, num_kv_heads, head_dim, page_size, out,
                              opts, g, rows);
    if (rc) return rc;
    const bool staged_ok = staged_strides_ok(k->stride[0], k->stride[1], g.P) &&
                           staged_strides_ok(v->stride[0], v->stride[1], g.P) && pa::prefill_staged_supported(head_dim);
    if (opts && opts->schedule == PA_SCHEDULE_STAGED && !staged_ok)
        return fail(PA_ENOTSUP, "staged schedule: head_dim 128/256, page stride < 2^32 and slot stride < 2^23 "
                    "elements");
    const PrefillPlan pl = plan_prefill(g, rows, opts, staged_ok);
    if ((int64_t)pl.n_slots * g.Hkv * pl.n_part > INT32_MAX) return fail(PA_ENOTSUP, "grid too large");
    if (!pl.staged && sizeof(int) * (size_t)(pa::lean_page_slots((int)g.P) + g.B + 1) >
                          pa::prefill_dynamic_lds_limit((int)g.D))
        return fail(PA_ENOTSUP, "head_dim %lld: %lld sequences of pages of %lld tokens leave no room in LDS",
                    (long long)g.D, (long long)g.B, (long long)g.P);
    if (rows == 0 || g.B == 0) return PA_OK;
    int ndev = 0, dev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(PA_ENODEV, "no HIP device");
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ENODEV, "hipGetDevice: %s", hipGetErrorString(e));
    void* ws = nullptr;
    if (pl.split) {
        if (workspace) {
            if (workspace_bytes < pl.ws_bytes)
                return fail(PA_ENOMEM, "workspace of %zu bytes, %zu needed", workspace_bytes, pl.ws_bytes);
            if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
                return fail(PA_EALIGN, "workspace not %zu-byte aligned", kAlign);
            ws = workspace;
        } else {
            rc = library_workspace(dev, pl.ws_bytes, static_cast<hipStream_t>(stream), &ws);
            if (rc) return rc;
        }
    }
    pa::DecodeParams p{};
    p.q = q->data;
    p.q_dtype = g.q_dtype;
    p.out_dtype = g.out_dtype;
    p.q_sb = q->stride[0];
    p.q_sh = q->stride[1];
    p.k = k->data;
    p.k_sp = k->stride[0];
    p.k_ss = k->stride[1];
    p.k_sh = k->stride[2];
    p.v = v->data;
    p.v_sp = v->stride[0];
    p.v_ss = v->stride[1];
    p.v_sh = v->stride[2];
    p.bt = static_cast<const int32_t*>(bt->data);
    p.bt_sb = bt->stride[0];
    p.ctx = static_cast<const int32_t*>(ctx->data);
    p.qstart = static_cast<const int32_t*>(qs->data);
    p.q_rows = (int)rows;
    p.n_slots = pl.n_slots;
    p.out = out->data;
    p.o_sb = out->stride[0];
    p.o_sh = out->stride[1];
    p.part_o = pl.split ? reinterpret_cast<float*>(static_cast<char*>(ws) + pl.o_offset) : nullptr;
    p.part_lse = pl.split ? reinterpret_cast<float*>(static_cast<char*>(ws) + pl.lse_offset) : nullptr;
    p.B = (int)g.B;
    p.Hq = (int)g.Hq;
    p.Hkv = (int)g.Hkv;
    p.P = (int)g.P;
    p.p_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((int64_t)1 << sh == g.P) p.p_shift = sh;
    p.max_blk = (int)g.max_blk;
    p.num_pages = (int)std::max<int64_t>(g.NP, 1);
    p.part_tokens = pl.part_tokens;
    p.n_part = pl.n_part;
    p.qw = 16;
    p.lean_page_slots = pa::lean_page_slots(p.P);
    p.window = opts ? opts->window : 0;
    p.scale_log2 = effective_scale(scale, g.D) * pa::kLog2e;
    e = pl.staged ? pa::launch_prefill_staged(p, (int)g.D, g.kv_dtype, static_cast<hipStream_t>(stream))
                  : pa::launch_prefill(p, (int)g.D, g.kv_dtype, pl.split, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_EHIP, "several-query launch: %s", hipGetErrorString(e));
    g_stats.prefill++;
    g_stats.last_schedule = pl.staged ? PA_SCHEDULE_STAGED : PA_SCHEDULE_PARTITIONS;
    if (pl.split) g_stats.merge++;
    g_stats.last_t = (uint64_t)pl.part_tokens;
    g_stats.last_np = (uint64_t)pl.n_part;
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_prefill(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
               const pa_tensor* block_tables, const pa_tensor* context_lens, const pa_tensor* query_start,
               float scale, int num_q_heads, int num_kv_heads, int head_dim, int page_size,
               const pa_tensor* out, void* stream, const pa_opts* opts, void* workspace,
               size_t workspace_bytes) {
    return prefill_impl(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, num_q_heads,
                        num_kv_heads, head_dim, page_size, out, stream, opts, workspace, workspace_bytes);
}

size_t pa_prefill_workspace_bytes(int64_t num_rows, int64_t num_seqs, int num_q_heads, int num_kv_heads,
                                  int head_dim, int64_t max_blocks_per_seq, int page_size,
                                  const pa_opts* opts) {
    if (num_rows < 0 || num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads ||
        head_dim < 1 || max_blocks_per_seq < 0 || page_size < 1)
        return 0;
    const int qg = num_q_heads / num_kv_heads;
    if (16 % qg) return 0;
    if (opts && (opts->partition_tokens < 0 || opts->window < 0)) return 0;
    Geometry g{num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, 1, max_blocks_per_seq, qg,
               PA_DTYPE_BF16, PA_DTYPE_BF16, PA_DTYPE_BF16};
    // An upper bound over the pool's strides: with strides the staged kernel
    // cannot take, the automatic schedule runs on partitions (and the staged
    // one fails).
    if (opts && opts->schedule == PA_SCHEDULE_STAGED) return plan_prefill(g, num_rows, opts, true).ws_bytes;
    return std::max(plan_prefill(g, num_rows, opts, true).ws_bytes, plan_prefill(g, num_rows, opts, false).ws_bytes);
}


int pa_cache_append(const pa_tensor* k_new, const pa_tensor* v_new, const pa_tensor* k_cache,
                    const pa_tensor* v_cache, const pa_tensor* block_tables,
                    const pa_tensor* context_lens, int num_kv_heads, int head_dim, int page_size,
                    void* stream) {
    t_err.clear();
    int rc = validate_append(k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                             head_dim, page_size);
    if (rc) return rc;
    if (k_new->shape[0] == 0) return PA_OK;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(PA_ENODEV, "no HIP device");
    pa::AppendParams a{};
    const int es = elem_size(k_cache->dtype);     // strides become byte strides
    a.k_new = static_cast<const char*>(k_new->data);
    a.v_new = static_cast<const char*>(v_new->data);
    a.kn_sb = k_new->stride[0] * es;
    a.kn_sh = k_new->stride[1] * es;
    a.vn_sb = v_new->stride[0] * es;
    a.vn_sh = v_new->stride[1] * es;
    a.k = static_cast<char*>(k_cache->data);
    a.v = static_cast<char*>(v_cache->data);
    a.k_sp = k_cache->stride[0] * es;
    a.k_ss = k_cache->stride[1] * es;
    a.k_sh = k_cache->stride[2] * es;
    a.v_sp = v_cache->stride[0] * es;
    a.v_ss = v_cache->stride[1] * es;
    a.v_sh = v_cache->stride[2] * es;
    a.bt = static_cast<const int32_t*>(block_tables->data);
    a.bt_sb = block_tables->stride[0];
    a.ctx = static_cast<const int32_t*>(context_lens->data);
    a.B = (int)k_new->shape[0];
    a.Hkv = num_kv_heads;
    a.row_bytes = head_dim * es;
    a.P = page_size;
    a.max_blk = (int)block_tables->shape[1];
    a.num_pages = (int)k_cache->shape[0];
    hipError_t e = pa::launch_append(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_EHIP, "append launch: %s", hipGetErrorString(e));
    g_stats.append++;
    return PA_OK;
}


int pa_decode(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
              const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
              int num_q_heads, int num_kv_heads, int head_dim, int page_size, const pa_tensor* out,
              void* stream) {
    return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, num_q_heads,
                       num_kv_heads, head_dim, page_size, out, stream, nullptr, nullptr, 0);
}

int pa_decode_ex(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                 const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                 int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                 const pa_tensor* out, void* stream, const pa_opts* opts, void* workspace,
                 size_t workspace_bytes) {
    return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, num_q_heads,
                       num_kv_heads, head_dim, page_size, out, stream, opts, workspace,
                       workspace_bytes);
}

int pa_decode_noalloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                      const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                      int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                      const pa_tensor* out, void* stream, const pa_opts* opts) {
    return decode_noalloc_impl(q, k_cache, v_cache, block_tables, context_lens, scale, num_q_heads,
                               num_kv_heads, head_dim, page_size, out, stream, opts);
}

int pa_check_args(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                  const pa_tensor* block_tables, const pa_tensor* context_lens, float scale,
                  int num_q_heads, int num_kv_heads, int head_dim, int page_size,
                  const pa_tensor* out, const pa_opts* opts) {
    t_err.clear();
    Geometry g;
    int rc = validate(q, k_cache, v_cache, block_tables, context_lens, scale, num_q_heads,
                      num_kv_heads, head_dim, page_size, out, opts, g);
    if (rc) return rc;
    Plan pl = make_plan(g, opts);
    rc = check_plan(g, pl, opts);
    if (rc) return rc;
    return PA_OK;
}

size_t pa_decode_workspace_bytes(int64_t num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int64_t max_blocks_per_seq, int page_size, const pa_opts* opts) {
    if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads ||
        head_dim < 1 || max_blocks_per_seq < 0 || page_size < 1)
        return 0;
    if (opts && opts->partition_tokens < 0) return 0;
    // The automatic variant depends on the K/V element type, which this
    // function is not told: return the larger of the two plans it can pick.
    Geometry g{num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, 1, max_blocks_per_seq,
               num_q_heads / num_kv_heads, PA_DTYPE_BF16, PA_DTYPE_BF16, PA_DTYPE_BF16};
    size_t bytes = make_plan(g, opts).ws_bytes;
    if (!opts || opts->variant == PA_VARIANT_AUTO) {
        Geometry g32 = g;
        g32.kv_dtype = PA_DTYPE_FP32;           // no MFMA path: the vector-ALU plan
        bytes = std::max(bytes, make_plan(g32, opts).ws_bytes);
    }
    return bytes;
}

int pa_get_stats(pa_stats* s) {
    if (!s) return PA_EINVAL;
    s->calls = g_stats.calls;
    s->valu_launches = g_stats.valu;
    s->mfma_launches = g_stats.mfma;
    s->split_calls = g_stats.split;
    s->merge_launches = g_stats.merge;
    s->last_partition_tokens = g_stats.last_t;
    s->last_num_partitions = g_stats.last_np;
    s->last_variant = g_stats.last_variant;
    s->balanced_calls = g_stats.lean;
    s->append_launches = g_stats.append;
    s->prefill_launches = g_stats.prefill;
    s->last_schedule = g_stats.last_schedule;
    s->fused_calls = g_stats.fused;
    return PA_OK;
}

int pa_trace_set(void* buf, size_t bytes) {
    static_assert(PA_TRACE_WORDS == pa::kTraceWords, "trace record size");
    if (buf && (reinterpret_cast<uintptr_t>(buf) & 15u))
        return fail(PA_EINVAL, "pa_trace_set: the buffer must be 16-byte aligned");
    const size_t rec = sizeof(uint64_t) * PA_TRACE_WORDS;
    const size_t wgs = buf ? std::min<size_t>(bytes / rec, INT32_MAX) : 0;
    g_trace_wgs = (int)wgs;
    g_trace = wgs ? static_cast<uint64_t*>(buf) : nullptr;
    return PA_OK;
}

int pa_trace_clock_khz(int* khz) {
    if (!khz) return fail(PA_EINVAL, "pa_trace_clock_khz: khz is NULL");
    int dev = 0, n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) return fail(PA_ENODEV, "no HIP device");
    if (hipGetDevice(&dev) != hipSuccess) return fail(PA_EHIP, "hipGetDevice failed");
    const hipError_t e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return fail(PA_EHIP, "hipDeviceGetAttribute(WallClockRate): %s", hipGetErrorString(e));
    return PA_OK;
}

void pa_reset_stats(void) {
    g_stats.calls = 0;
    g_stats.valu = 0;
    g_stats.mfma = 0;
    g_stats.split = 0;
    g_stats.merge = 0;
    g_stats.lean = 0;
    g_stats.append = 0;
    g_stats.prefill = 0;
    g_stats.fused = 0;
    g_stats.last_schedule = 0;
    g_stats.last_t = 0;
    g_stats.last_np = 0;
    g_stats.last_variant = 0;
}

const char* pa_strerror(int code) {
    switch (code) {
        case PA_OK: return "success";
        case PA_EINVAL: return "invalid argument";
        case PA_ENOTSUP: return "unsupported configuration";
        case PA_EALIGN: return "misaligned pointer or stride";
        case PA_ENODEV: return "no HIP device";
        case PA_ENOMEM: return "out of memory or workspace too small";
        case PA_EHIP: return "HIP runtime error";
        default: return "unknown error code";
    }
}

const char* pa_last_error(void) { return t_err.c_str(); }

int pa_release(void) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int rc = PA_OK;
    int cur = -1;
    bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (size_t d = 0; d < g_ws.size(); ++d) {
        Workspace& w = g_ws[d];
        if (!w.ptr && w.retired.empty()) continue;
        bool ok = hipSetDevice((int)d) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
        for (void* r : w.retired) ok = ok && hipFree(r) == hipSuccess;
        if (w.ptr) ok = ok && hipFree(w.ptr) == hipSuccess;
        if (!ok) rc = fail(PA_EHIP, "releasing workspace of device %zu failed", d);
        w.ptr = nullptr;
        w.bytes = 0;
        w.retired.clear();
    }
    if (have_cur) (void)hipSetDevice(cur);
    return rc;
}

const char* pa_version(void) { return "0.1.0"; }

}  // extern "C"
