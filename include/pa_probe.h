/*
 * pa_probe.h -- streaming-read probes: the bandwidth references the decode
 * kernels are measured against (libpa_probe.so, built beside
 * libpa_decode.so).  Measurement aids, not part of the attention library.
 *
 * Each probe only reads: it streams the bytes a decode call would read, with
 * no arithmetic, so its rate is what the memory system gives that access
 * pattern.  Two patterns (and an issue-rate probe, below):
 *
 *  - contiguous: `bytes` bytes from `base`, 16 bytes per lane per load,
 *    grid-stride over n_wg workgroups of 256 threads;
 *  - paged: the K and V rows of every (sequence, KV head, token) of a paged
 *    NHD cache, read through the block table -- the decode's own pattern
 *    (page 1 of the source pages, issue "ROCm gfx1200: PagedAttnOnline is
 *    8.1x slower per call", section "Where to look": NHD KV addressed
 *    through strides and a block table).  The (sequence, KV head, 16-token
 *    tile) work is cut into n_wg equal shares, one per workgroup of four
 *    waves, each wave keeping two (head_dim 256) or three (128) tiles of
 *    loads in flight, as the matrix-core decode kernel does.
 *
 * The loaded words are folded into one value per thread; `sink` (device
 * memory of n_wg 32-bit words) is written only if that value equals a fixed
 * constant, so the loads cannot be dropped and nothing else is written.
 * Calls are asynchronous on `stream` (a hipStream_t, NULL = null stream).
 * Return 0 on success, 1 on a bad argument (nothing enqueued), 2 when the
 * launch failed.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* base: device pointer, 16-byte aligned; bytes: a multiple of 16;
 * n_wg: 1 .. 65536. */
int pa_probe_read_contiguous(const void* base, int64_t bytes, int n_wg, void* sink, void* stream);

typedef struct pa_probe_paged {
    const void* k;               /* [NP, P, Hkv, D] pools (device), any 16-byte element type */
    const void* v;
    int64_t k_sp, k_ss, k_sh;    /* byte strides of page, slot, KV head; multiples of 16 */
    int64_t v_sp, v_ss, v_sh;
    int32_t row_bytes;           /* bytes of one (token, KV head) row: 256 or 512      */
    const int32_t* block_tables; /* [B, MaxBlk] int32 (device)                         */
    int64_t bt_sb;               /* row stride of block_tables, in elements            */
    const int32_t* context_lens; /* [B] int32 (device)                                 */
    int32_t batch;               /* B, 1 .. 4096                                       */
    int32_t num_kv_heads;        /* Hkv >= 1                                           */
    int32_t page_size;           /* P: a power of two >= 16                            */
    int32_t num_pages;           /* NP >= 1: page ids are clamped into [0, NP)         */
    int32_t max_blocks;          /* MaxBlk >= 1: lengths are clamped to MaxBlk * P     */
} pa_probe_paged;

/* n_wg: 1 .. 4096 workgroups. */
int pa_probe_read_paged(const pa_probe_paged* d, int n_wg, void* sink, void* stream);

/* Issue-rate probe of one CU's SIMDs (no memory traffic): how matrix-core
 * products and vector-ALU work share a SIMD, the bound of the several-query
 * kernel, whose 32-token pairs issue 26 MFMAs and about 64 other VALU
 * instructions in dependent blocks.  Mode i of a fixed menu runs `rounds`
 * rounds of NM 16x16x32 bf16 MFMAs and NV independent fp32 FMAs per wave,
 * either interleaved in every wave (mixed = 1) or split between MFMA-only and
 * FMA-only waves (mixed = 0); n_wg workgroups of 256 threads (on 256 CUs,
 * 256 of them give one wave per SIMD and 1024 give four).  The caller times
 * the launch.
 *
 * pa_probe_issue_modes(i, &nm, &nv, &mixed): describes mode i; returns the
 * number of modes (also for i < 0, which writes nothing), -1 for i past the
 * menu or a NULL output.
 * pa_probe_issue: 0 on success, 1 on a bad argument (mode outside the menu,
 * n_wg outside 1 .. 65536, rounds outside 1 .. 2^20, sink NULL; nothing
 * enqueued), 2 when the launch failed.  sink: n_wg 32-bit words (device). */
int pa_probe_issue_modes(int mode, int* nm, int* nv, int* mixed);
int pa_probe_issue(int mode, int n_wg, int rounds, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
