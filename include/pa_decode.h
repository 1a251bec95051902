/*
 * pa_decode.h -- C ABI of the MI355X (gfx950) decode paged-attention library.
 *
 * One operation: single-query (decode) attention of every sequence's newest
 * query over that sequence's keys and values, read page by page from an NHD
 * paged KV cache through a block table.
 *
 *   Source: page 1 of the source pages, issue "ROCm gfx1200: PagedAttnOnline
 *   is 8.1x slower per call than vLLM's paged-attention kernel", section
 *   "Where to look" (online softmax, NHD KV addressed through strides,
 *   device-side request lookup); page 2, PR "head_dim=128 decode arm", section
 *   "Correctness" (bf16, grouped-query attention, head_dim 128); page 3, PR
 *   "head_dim-128 arm for the warp-split-KV decode kernel" (split-KV decode,
 *   the numerics table's 32-token pages).
 *
 * For sequence b (L = context_lens[b] tokens) and query head h, with
 * qg = num_q_heads / num_kv_heads and g = h / qg:
 *
 *   token t is stored at  page = block_tables[b][t / page_size],
 *                         slot = t % page_size,
 *   x_t  = scale * dot(q[b][h][:], k_cache[page][slot][g][:])
 *   out[b][h][:] = sum_t softmax(x)_t * v_cache[page][slot][g][:]
 *
 * over t in [0, L), or with a sliding window of W tokens (pa_opts.window)
 * over t in [max(0, L - W), L).  Q, the K/V cache and out are each bf16,
 * IEEE binary16 or binary32 (K and V share one type).  Arithmetic is fp32
 * (online softmax, fp32 accumulation; on the matrix cores the products take
 * Q and P in the cache's 16-bit type, P as the sum of two such values); the
 * output is rounded to its type, nearest even.  L == 0 writes zeros.  There
 * is no mask other than the window and no positional term.
 *
 * All functions are plain C, never throw, and make no HIP call before their
 * arguments have been validated.  Calls are asynchronous on the given stream:
 * a PA_OK return means the work was enqueued; device faults surface at the
 * caller's next synchronisation.  The library keeps no reference to caller
 * memory after a call returns, but the caller must keep every tensor alive
 * until the enqueued work has finished.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- errors */
#define PA_OK       0  /* success                                                  */
#define PA_EINVAL   1  /* null pointer, bad shape/dtype/stride, Hq % Hkv != 0,
                          infinite scale, page_size < 1, a library workspace
                          asked for on a stream under capture                      */
#define PA_ENOTSUP  2  /* head_dim not 128/256/512, Hq/Hkv not 1, 2, 4, 8 or 16, or a
                          kernel/schedule that does not take the call's shape      */
#define PA_EALIGN   3  /* a base pointer or a row stride not 16-byte aligned       */
#define PA_ENODEV   4  /* no HIP device available                                  */
#define PA_ENOMEM   5  /* workspace could not be allocated, or is too small        */
#define PA_EHIP     6  /* a HIP runtime call failed; text in pa_last_error()        */

/* The scale argument's request for the default 1/sqrt(head_dim). */
#define PA_SCALE_DEFAULT (__builtin_nanf(""))

/* ---------------------------------------------------------------- tensors */
#define PA_DTYPE_BF16  1
#define PA_DTYPE_INT32 2
#define PA_DTYPE_FP32  3
#define PA_DTYPE_F16   4   /* IEEE binary16 */

/*
 * A strided view of device memory.  shape[] and stride[] are in elements;
 * entries at index >= ndim are ignored.  The library only reads the
 * descriptor during the call.
 */
typedef struct pa_tensor {
    void*   data;       /* device pointer                                    */
    int32_t dtype;      /* PA_DTYPE_*                                        */
    int32_t ndim;
    int64_t shape[4];
    int64_t stride[4];
} pa_tensor;

/*
 * pa_decode -- enqueue one decode paged-attention call.
 *
 *  q             [B, Hq, D]        bf16, fp16 or fp32; stride[2] == 1;
 *                                  stride[0], stride[1] multiples of 16 bytes.
 *  k_cache       [NP, P, Hkv, D]   NHD pool (page, slot, KV head, dim) of
 *                                  bf16, fp16 or fp32; stride[3] == 1, other
 *                                  strides multiples of 16 bytes.  Pages may
 *                                  lie anywhere in the pool: block_tables
 *                                  gives the order.
 *  v_cache       same shape and element type as k_cache (its own strides,
 *                same rules).
 *  block_tables  [B, MaxBlk]       int32, stride[1] == 1.  Entry j of row b is
 *                                  the physical page of tokens
 *                                  [j*P, (j+1)*P) of sequence b.  Entries at
 *                                  or past ceil(L_b / P) are never read and
 *                                  may hold anything (e.g. -1).
 *  context_lens  [B]               int32, stride[0] == 1.  L_b tokens.
 *  scale         fp32 multiplier of the logits, or PA_SCALE_DEFAULT (a NaN)
 *                for the method's 1/sqrt(D) (the fp32 value nearest to it).
 *                An infinite scale is PA_EINVAL.
 *  num_q_heads, num_kv_heads, head_dim, page_size
 *                must equal q.shape[1], k_cache.shape[2], q.shape[2] and
 *                k_cache.shape[1].
 *  out           [B, Hq, D]        bf16, fp16 or fp32, stride[2] == 1,
 *                                  16-byte aligned rows.
 *  stream        hipStream_t to enqueue on; NULL is the null stream.
 *
 * Device-side preconditions, not checked on the host (the host never reads
 * device memory): 0 <= L_b <= MaxBlk * P and every used block-table entry is
 * in [0, NP).  The kernels clamp L_b into [0, MaxBlk * P] and page ids into
 * [0, NP), so a violation gives unspecified output, never an out-of-range
 * access.
 *
 * Work is split over workgroups either as fixed-size partitions of each
 * sequence or, on the MFMA variant, as equal shares of all sequences' work
 * (chosen automatically for large calls: at most 4096 sequences and at
 * least 262144 units of (sequence, query block, 16 tokens of capacity
 * MaxBlk * P, or of the window)), or as partitions whose size the kernel
 * fits to the actual lengths (chosen automatically, without a window and
 * for at most 256 sequences, where fixed partitions would cut the tables
 * into 4 or more and the tables hold at least 192 MB of K/V); partial results are
 * merged with the log-sum-exp rule by a second kernel or, where that is
 * faster (fixed partitions, at most two per (sequence, query block), at
 * most 256 workgroups; pa_opts.merge), inside the decode kernel by the last
 * partition of each group to finish.  The library keeps a
 * per-device workspace for the partials, grown on demand with hipMalloc
 * (an outgrown buffer is kept until pa_release(), which frees them all);
 * calls that use it must not overlap in time on one device (callers that
 * overlap calls pass their own workspaces to pa_decode_ex).  A call on a
 * stream that is being captured into a graph cannot use that workspace and
 * returns PA_EINVAL (captured calls use pa_decode_ex with a workspace, or
 * pa_decode_noalloc).  Returns PA_OK or an error code above.
 */
int pa_decode(const pa_tensor* q,
              const pa_tensor* k_cache,
              const pa_tensor* v_cache,
              const pa_tensor* block_tables,
              const pa_tensor* context_lens,
              float scale,
              int num_q_heads,
              int num_kv_heads,
              int head_dim,
              int page_size,
              const pa_tensor* out,
              void* stream);

/*
 * pa_cache_append -- enqueue the KV-cache write of every sequence's newest
 * token: the step that precedes pa_decode in a decode step.  Not on the
 * source pages (their kernels only read the cache); the plainest neighbour of
 * the decode step, on the same NHD pool (page 1, issue "ROCm gfx1200:
 * PagedAttnOnline is 8.1x slower per call", section "Where to look").
 *
 *  k_new, v_new  [B, Hkv, D]        bf16, fp16 or fp32 (the caches' type),
 *                                   stride[2] == 1, 16-byte aligned rows.
 *  k_cache, v_cache [NP, P, Hkv, D] NHD pools of one element type, as in
 *                pa_decode; written (the rows are copied bit for bit).
 *  block_tables  [B, MaxBlk] int32; context_lens [B] int32 -- lengths that
 *                already count the new token.
 *  num_kv_heads, head_dim, page_size must equal the shapes; a row of head_dim
 *                elements must be whole 16-byte chunks (PA_ENOTSUP else).
 *
 * For each b with L = context_lens[b] >= 1 and t = L - 1, the rows
 * k_new[b][g][:] and v_new[b][g][:] of every KV head g are written to
 * k_cache / v_cache[block_tables[b][t / P]][t % P][g][:].  L <= 0 writes
 * nothing.  Device-side preconditions, not checked on the host: L <= MaxBlk * P
 * and that page id in [0, NP); a sequence that violates them writes nothing.
 * Sequences whose newest tokens share a slot race (one of them wins).
 * Asynchronous on the stream; returns PA_OK or an error code.
 */
int pa_cache_append(const pa_tensor* k_new,
                    const pa_tensor* v_new,
                    const pa_tensor* k_cache,
                    const pa_tensor* v_cache,
                    const pa_tensor* block_tables,
                    const pa_tensor* context_lens,
                    int num_kv_heads,
                    int head_dim,
                    int page_size,
                    void* stream);

/* ---------------------------------------------------------------- options */
#define PA_VARIANT_AUTO  0   /* the library picks                              */
#define PA_VARIANT_VALU  1   /* vector-ALU kernel (any supported qg)            */
#define PA_VARIANT_MFMA  2   /* matrix-core kernel (bf16 or fp16 MFMA for Q.K
                                and P.V; 16-bit caches, head_dim 128/256/512;
                                the balanced schedule at 128/256 only)        */

#define PA_SCHEDULE_AUTO        0  /* the library picks                         */
#define PA_SCHEDULE_PARTITIONS  1  /* one workgroup per fixed-size partition of
                                      each sequence (split-KV partitions)      */
#define PA_SCHEDULE_BALANCED    2  /* MFMA only: the work of all sequences cut
                                      into one equal static share per
                                      workgroup plus small units taken from a
                                      counter as workgroups finish           */
#define PA_SCHEDULE_STAGED      3  /* pa_prefill only: a workgroup takes eight
                                      query blocks of one sequence, which share
                                      every K/V stage through LDS; no split   */
#define PA_SCHEDULE_FITTED      4  /* MFMA only, no window, at most 256
                                      sequences, MaxBlk * P < 2^24 tokens:
                                      split-KV partitions whose size
                                      the kernel picks per call from the
                                      context lengths, so that the partitions
                                      fill `shares` workgroups (0 = one per
                                      compute unit); partitions of no work are
                                      never launched.  The workspace keeps, per
                                      workgroup, the partition it took in the
                                      last call as a starting guess for the
                                      next; any content there is valid.       */

/* How split partitions are merged (log-sum-exp): */
#define PA_MERGE_AUTO    0   /* the library picks                              */
#define PA_MERGE_KERNEL  1   /* a second kernel merges them after the decode   */
#define PA_MERGE_FUSED   2   /* inside the decode kernel: the last partition of
                                each (sequence, query block) group to finish
                                merges the group's partials (MFMA variant,
                                partition or fitted schedule, at most
                                PA_FUSE_MAX_GROUPS groups)                     */
#define PA_FUSE_MAX_GROUPS 16320

typedef struct pa_opts {
    int32_t variant;            /* PA_VARIANT_*                                */
    int32_t partition_tokens;   /* 0 = automatic; else tokens per split-KV
                                   partition, a multiple of 64 (rounded up).
                                   A value >= MaxBlk * P disables the split.
                                   Setting it selects the partition schedule
                                   unless schedule says otherwise.             */
    int32_t schedule;           /* PA_SCHEDULE_*                               */
    int32_t shares;             /* balanced schedule: 0 = automatic (one per
                                   compute unit at most), else the number of
                                   workgroups, 1 .. 1024                       */
    int32_t window;             /* sliding window: 0 = attend to all L tokens;
                                   W >= 1 = only the last W, tokens
                                   [max(0, L - W), L) (page 3, LIMITATIONS,
                                   the windowed variant)                       */
    int32_t merge;              /* PA_MERGE_*                                  */
    int32_t reserved[2];        /* must be zero                                */
} pa_opts;

/*
 * Bytes of workspace pa_decode_ex needs for a call with these sizes and
 * options (0 when the call does not split).  max_blocks_per_seq is
 * block_tables.shape[1].  With the automatic variant the kernel depends on
 * the K/V element type, which is not an argument here: the result is then
 * the larger of the two plans, enough for any element type.  Returns 0 on
 * bad arguments as well.
 */
#define PA_WORKSPACE_ZERO_BYTES 65536
size_t pa_decode_workspace_bytes(int64_t num_seqs, int num_q_heads, int num_kv_heads,
                                 int head_dim, int64_t max_blocks_per_seq, int page_size,
                                 const pa_opts* opts);

/*
 * pa_decode_ex -- pa_decode with options and caller-owned workspace.
 * opts may be NULL (automatic).  workspace is a device buffer of at least
 * pa_decode_workspace_bytes(...) bytes, 256-byte aligned, owned by the caller
 * and in use until the enqueued work finishes; if workspace is NULL the
 * library's own per-device workspace is used (as in pa_decode).  Its first
 * PA_WORKSPACE_ZERO_BYTES hold work and arrival counters: they must be zero
 * before the workspace's first use (e.g. allocate it zeroed), and every call
 * leaves them zero, so a workspace can be reused by any later call of any
 * schedule.  Returns PA_ENOMEM if the given workspace is too small.
 */
int pa_decode_ex(const pa_tensor* q,
                 const pa_tensor* k_cache,
                 const pa_tensor* v_cache,
                 const pa_tensor* block_tables,
                 const pa_tensor* context_lens,
                 float scale,
                 int num_q_heads,
                 int num_kv_heads,
                 int head_dim,
                 int page_size,
                 const pa_tensor* out,
                 void* stream,
                 const pa_opts* opts,
                 void* workspace,
                 size_t workspace_bytes);

/*
 * pa_decode_noalloc -- pa_decode_ex (workspace NULL aside) for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Not an operation of the source
 * pages: the same decode, whose split-KV partials, work counters and
 * partition hints go to a static per-device scratch array of
 * PA_NOALLOC_SCRATCH_BYTES inside the library instead of a workspace.
 *
 * Arguments, layouts and results as pa_decode_ex with opts (may be NULL).
 * Makes no hipMalloc / hipFree call.  A call whose split-KV plan needs more
 * scratch than PA_NOALLOC_SCRATCH_BYTES (pa_decode_workspace_bytes tells,
 * for the call's variant) returns PA_ENOMEM before any launch.  Each device
 * the library runs on holds the array from its first pa_decode_noalloc call
 * until the process ends.  That first call on a device sets the scratch up
 * (looks up its address, clears its work counters on the call's stream) and
 * must not be captured (PA_EINVAL); later calls may be.  Every call on one
 * device shares that device's array: calls that overlap in time on one
 * device (other streams, other threads, graphs replayed concurrently) race
 * and give unspecified results.  Every call leaves the work counters zero.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_noalloc(const pa_tensor* q,
                      const pa_tensor* k_cache,
                      const pa_tensor* v_cache,
                      const pa_tensor* block_tables,
                      const pa_tensor* context_lens,
                      float scale,
                      int num_q_heads,
                      int num_kv_heads,
                      int head_dim,
                      int page_size,
                      const pa_tensor* out,
                      void* stream,
                      const pa_opts* opts);

/*
 * pa_check_args -- run only the host-side validation of pa_decode_ex and
 * return the code it would return before touching the GPU (PA_OK if the
 * arguments are acceptable).  Makes no HIP call.
 */
int pa_check_args(const pa_tensor* q,
                  const pa_tensor* k_cache,
                  const pa_tensor* v_cache,
                  const pa_tensor* block_tables,
                  const pa_tensor* context_lens,
                  float scale,
                  int num_q_heads,
                  int num_kv_heads,
                  int head_dim,
                  int page_size,
                  const pa_tensor* out,
                  const pa_opts* opts);

/*
 * pa_prefill -- several queries per sequence: chunked prefill, or a batch
 * that mixes prefill chunks with decode steps.  (The pages name vLLM's
 * chunked-prefill paged-decode path -- page 1, issue "ROCm gfx1200:
 * PagedAttnOnline is 8.1x slower per call", section "Where to look" -- and
 * owe d=128 prefill -- page 2, PR "head_dim=128 decode arm", "Not
 * claimed".)
 *
 *  q             [R, Hq, D]       the query rows of all sequences, bf16, fp16
 *                                 or fp32; sequence b's rows are
 *                                 [query_start[b], query_start[b+1]).
 *  query_start   [B + 1] int32    0 = query_start[0] <= ... <= query_start[B] = R.
 *  k_cache, v_cache, block_tables [B, MaxBlk], context_lens [B]: as in
 *                pa_decode; context_lens already count the queried tokens.
 *  out           [R, Hq, D]       bf16, fp16 or fp32.
 *  opts          may be NULL; window and partition_tokens apply; the variant
 *                must be automatic or MFMA.  Schedules: PARTITIONS = one
 *                workgroup per query block (16 / qg query tokens times the
 *                qg heads of a KV head), long contexts split into partitions
 *                merged by log-sum-exp; STAGED = eight consecutive query
 *                blocks per workgroup share each K/V stage (no split, no
 *                workspace; partition_tokens must be 0); AUTO takes STAGED
 *                when partition_tokens is 0, the call has at least two query
 *                blocks per sequence on average and the staged grid has at
 *                least 256 workgroups, else PARTITIONS.  BALANCED is
 *                PA_ENOTSUP.
 *
 * Sequence b's n_b = query_start[b+1] - query_start[b] queries are its last
 * n_b tokens: query i sits at position pos = L_b - n_b + i and attends to the
 * tokens [0, pos] (with a window W: [max(0, pos - W + 1), pos]).  n_b = 1 is
 * the decode of pa_decode.  Runs on the matrix cores only: head_dim 128, 256
 * or 512 (STAGED: 128 or 256) and a bf16 or fp16 cache (else PA_ENOTSUP), at
 * most 4096 sequences (at head_dim 512 fewer when the pages are very small:
 * the per-block kernel keeps a fill of page ids and the sequences' block
 * counts in LDS beside its merge buffer; PA_ENOTSUP past that).
 * Device-side preconditions, not checked on the host: query_start as above
 * and n_b <= L_b (a query at a negative position gives zeros).  Workspace
 * rules as in pa_decode_ex (workspace NULL = the library's own).
 */
int pa_prefill(const pa_tensor* q,
               const pa_tensor* k_cache,
               const pa_tensor* v_cache,
               const pa_tensor* block_tables,
               const pa_tensor* context_lens,
               const pa_tensor* query_start,
               float scale,
               int num_q_heads,
               int num_kv_heads,
               int head_dim,
               int page_size,
               const pa_tensor* out,
               void* stream,
               const pa_opts* opts,
               void* workspace,
               size_t workspace_bytes);

/* Bytes of workspace pa_prefill needs for num_rows query rows over num_seqs
 * sequences (0 when the call does not split; 0 on bad arguments). */
size_t pa_prefill_workspace_bytes(int64_t num_rows, int64_t num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int64_t max_blocks_per_seq,
                                  int page_size, const pa_opts* opts);

/* ----------------------------------------------------- introspection */
/* Launch counters since load or the last pa_reset_stats (process-wide). */
typedef struct pa_stats {
    uint64_t calls;             /* successful pa_decode / pa_decode_ex calls   */
    uint64_t valu_launches;     /* decode-kernel launches, vector-ALU variant  */
    uint64_t mfma_launches;     /* decode-kernel launches, MFMA variant        */
    uint64_t split_calls;       /* calls that split the context                */
    uint64_t merge_launches;    /* log-sum-exp merge kernel launches           */
    uint64_t last_partition_tokens; /* partition size of the last call (0 on the
                                       balanced schedule)                      */
    uint64_t last_num_partitions;   /* partitions of the last call, or shares
                                       (workgroups) on the balanced schedule   */
    uint64_t last_variant;          /* PA_VARIANT_* of the last call           */
    uint64_t balanced_calls;        /* calls run on the balanced schedule      */
    uint64_t last_schedule;         /* PA_SCHEDULE_* of the last call          */
    uint64_t append_launches;       /* pa_cache_append kernel launches         */
    uint64_t prefill_launches;      /* pa_prefill kernel launches              */
    uint64_t fused_calls;           /* split calls merged inside the decode
                                       kernel (no merge kernel launched)      */
} pa_stats;

int  pa_get_stats(pa_stats* stats);   /* PA_EINVAL if stats is NULL            */
void pa_reset_stats(void);

/* Per-workgroup timeline of the matrix-core decode on fixed or fitted
 * partitions (a measurement aid, for instance to see start-up, streaming,
 * wave merge and in-kernel merge per CU).  While a buffer is set, every
 * launch of that kernel writes PA_TRACE_WORDS uint64 per workgroup for the
 * first bytes / (8 * PA_TRACE_WORDS) workgroups: [0] entry, [1] prologue done
 * (lengths, page ids, Q), [2] wave 0's streaming done, [3] wave merge and
 * stores done, [4] exit, in s_memrealtime ticks (pa_trace_clock_khz; [1]..[3] are 0 for
 * a workgroup with no partition to run); [5] HW_ID | XCC_ID << 32; [6]
 * sequence | query block << 16 | partition << 32; [7] partition tokens |
 * flags << 32 (1: no partition to run, 2: merged its group in the kernel).
 * Each launch overwrites the records; graphs captured while a buffer is set
 * keep writing to it.  buf: device memory owned by the caller, 16-byte
 * aligned; NULL (or bytes < 64) stops tracing.  Process-wide, like the
 * counters.  Returns PA_OK, or PA_EINVAL for a misaligned buffer. */
#define PA_TRACE_WORDS 8
int  pa_trace_set(void* buf, size_t bytes);
/* Frequency of the records' clock on the current device, in kHz (the HIP
 * wall-clock rate).  PA_EINVAL if khz is NULL, PA_ENODEV / PA_EHIP if the
 * runtime cannot tell. */
int  pa_trace_clock_khz(int* khz);

/* Static text for an error code; never NULL. */
const char* pa_strerror(int code);

/* Detail of the calling thread's last error ("" if none); valid until the
 * thread's next call into the library. */
const char* pa_last_error(void);

/* Free the library-owned workspaces of all devices.  Synchronises each device
 * that has one.  Returns PA_OK or PA_EHIP. */
int pa_release(void);

/* Library version, e.g. "0.1.0". */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
