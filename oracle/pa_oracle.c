/*
 * pa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * The plain, slow, fp64 CPU definition of single-query (decode) paged
 * attention.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library; the product path never does.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes (page 1 of the source pages, issue "ROCm gfx1200:
 * PagedAttnOnline is 8.1x slower per call...", section "Where to look": an
 * online-softmax decode kernel reading an NHD KV cache through strides, with
 * a device-side request lookup, i.e. a block table; page 2, PR "head_dim=128
 * decode arm", section "Correctness": the CPU oracle at Qwen3 geometry, bf16,
 * GQA 2, head_dim 128).  Online softmax and split-KV only reorder the sums of
 * ordinary softmax attention, so the oracle is that plain definition:
 *
 *   for sequence b with L = context_lens[b] tokens and query head h,
 *   g = floor(h / (Hq / Hkv))                    (grouped-query sharing)
 *   token t lives in physical page  block_tables[b][floor(t / P)],
 *                     slot          t mod P
 *   x_t   = s * sum_i q[b][h][i] * K[page][slot][g][i]      (s = fp32 scale)
 *   m     = max_t x_t
 *   w_t   = exp(x_t - m),  Z = sum_t w_t
 *   o[i]  = (sum_t w_t * V[page][slot][g][i]) / Z
 *
 * Sliding window (page 3, PR "head_dim-128 arm for the warp-split-KV decode
 * kernel", LIMITATIONS, names a windowed variant without defining it): with
 * a window of W >= 1 tokens the query attends to the last W tokens only,
 * t in [max(0, L - W), L); W == 0 means no window.  This is the plainest
 * reading: the decode query sits at position L - 1 and sees itself and the
 * W - 1 tokens before it.
 *
 * Several queries per sequence (chunked prefill; page 1, "Where to look",
 * names vLLM's chunked-prefill paged-decode path; the pages owe d=128
 * prefill -- page 2, "Not claimed"): sequence b's n_b query rows are its
 * last n_b tokens, so query i sits at position pos = L - n_b + i and
 * attends causally to t in [0, pos] (with a window W: [max(0, pos-W+1),
 * pos]).  One query per sequence is the decode case above.
 *
 * Readings where the pages are silent: L == 0 gives an all-zero row; the
 * scale is the fp32 value the caller passes, widened exactly; there is no
 * mask other than the window, no soft-cap and no positional term.  Sums run
 * in ascending t and ascending i inside one (b, h) pair, so the result does
 * not depend on the number of threads.
 *
 * Every input is read as the exact value of its storage type widened to
 * fp64: bf16, IEEE binary16 or binary32 (element types of Q and of the K/V
 * pools are given separately).  Block-table entries of used pages are
 * range-checked; bad input returns an error code.
 *
 * The "mutant" argument exists only so that a test can plant a known mistake
 * in the oracle and show that the pins catch it.  0 is the definition.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_EPAGE -2
#define ORC_ENOMEM -3

#define ORC_BF16 1
#define ORC_F32 3
#define ORC_F16 4

typedef struct {
    const void* q;
    int64_t q_sb, q_sh;                 /* element strides of q [B][Hq][D]   */
    const void* k;
    const void* v;
    int q_dtype, kv_dtype;              /* ORC_BF16 / ORC_F16 / ORC_F32      */
    int64_t s_page, s_slot, s_head;     /* element strides of the NHD pools  */
    int64_t num_pages;
    const int32_t* bt;
    int64_t max_blk;
    const int32_t* ctx;
    int B, Hq, Hkv, D, P;
    double scale;
    int64_t window;                     /* 0 = none, else the last W tokens  */
    int mutant;
    /* several queries per sequence: rows [qstart[b], qstart[b+1]) of q */
    const int32_t* qstart;              /* NULL = one query per sequence     */
    int64_t n_rows;
    /* work list */
    const int32_t* pairs;               /* (b, h) pairs, or NULL = all       */
    int64_t n_items;
    double* out;                        /* [n_items][D]                      */
    int status;
} orc_args;

typedef struct {
    orc_args* a;
    int64_t begin, end;
    int status;
} orc_slice;

static double bf16_bits_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double f16_bits_to_f64(uint16_t h)
{
    int e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                  /* zero, subnormal */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);             /* (1 + m/2^10) 2^(e-15) */
    return (h & 0x8000) ? -v : v;
}

/* Element idx of an array of the given storage type, widened exactly. */
static double elem(const void* base, int64_t idx, int dtype)
{
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    if (dtype == ORC_F16) return f16_bits_to_f64(((const uint16_t*)base)[idx]);
    return bf16_bits_to_f64(((const uint16_t*)base)[idx]);
}

/* One output row o[0..D) following the definition above: query row qoff of
 * q, head h, attending to tokens [.., L) of sequence b (L = the position of
 * the query plus one). */
static int attend(const orc_args* a, int b, int64_t qoff, int64_t L, int h, double* o)
{
    const int D = a->D;
    for (int i = 0; i < D; ++i) o[i] = 0.0;
    if (L <= 0) return ORC_OK;
    if (L > a->max_blk * a->P) return ORC_EINVAL;

    const int qg = a->Hq / a->Hkv;
    int g = h / qg;
    if (a->mutant == 1) g = h % a->Hkv;            /* wrong head map          */

    if (a->mutant == 10 && a->qstart && L < a->max_blk * a->P) L += 1;   /* sees one token ahead */
    /* first attended token: the window keeps t >= L - W */
    int64_t t0 = (a->window > 0 && L > a->window) ? L - a->window : 0;
    if (a->mutant == 9 && a->window > 0 && L > a->window) t0 += 1;   /* window one short */

    double* x = (double*)malloc((size_t)L * sizeof(double));
    int64_t* voff = (int64_t*)malloc((size_t)L * sizeof(int64_t));
    const void** vbase = (const void**)malloc((size_t)L * sizeof(void*));
    if (!x || !voff || !vbase) { free(x); free(voff); free(vbase); return ORC_ENOMEM; }

    for (int64_t t = t0; t < L; ++t) {
        int64_t lp = t / a->P, slot = t % a->P;
        if (a->mutant == 2) slot = (t + 1) % a->P;        /* off-by-one slot */
        if (lp >= a->max_blk) { free(x); free(voff); free(vbase); return ORC_EPAGE; }
        int64_t page = a->bt[(int64_t)b * a->max_blk + lp];
        if (a->mutant == 8) page = a->bt[lp];             /* batch row lost  */
        if (page < 0 || page >= a->num_pages) { free(x); free(voff); free(vbase); return ORC_EPAGE; }
        int64_t off = page * a->s_page + slot * a->s_slot + (int64_t)g * a->s_head;
        voff[t] = off;
        vbase[t] = a->v;
        if (a->mutant == 5) vbase[t] = a->k;               /* K used in place of V */
        double dot = 0.0;
        for (int i = 0; i < D; ++i) {
            double qi = elem(a->q, qoff + i, a->q_dtype);
            double ki = elem(a->k, off + i, a->kv_dtype);
            if (a->mutant == 6 && i == D - 1) ki = 0.0;   /* dropped term    */
            dot += qi * ki;
        }
        x[t] = a->scale * dot;
        if (a->mutant == 3) x[t] = dot;                   /* scale ignored   */
        if (a->mutant == 4) x[t] = -a->scale * dot;       /* wrong sign      */
    }

    double m = -INFINITY;
    for (int64_t t = t0; t < L; ++t) if (x[t] > m) m = x[t];
    double Z = 0.0;
    for (int64_t t = t0; t < L; ++t) {
        x[t] = exp(x[t] - m);                             /* x now holds w_t */
        Z += x[t];
    }
    int64_t t_end = L;
    if (a->mutant == 7) t_end = L - 1;                    /* last token lost */
    for (int64_t t = t0; t < t_end; ++t)
        for (int i = 0; i < D; ++i) o[i] += x[t] * elem(vbase[t], voff[t] + i, a->kv_dtype);
    for (int i = 0; i < D; ++i) o[i] /= Z;

    free(x);
    free(voff);
    free(vbase);
    return ORC_OK;
}

/* Decode: sequence b's one query q[b][h] over all L_b tokens. */
static int attend_row(const orc_args* a, int b, int h, double* o)
{
    return attend(a, b, (int64_t)b * a->q_sb + (int64_t)h * a->q_sh, a->ctx[b], h, o);
}

/* Several queries: query row r (of sequence b, found from qstart) over
 * [.., pos + 1). */
static int attend_query(const orc_args* a, int64_t r, int h, double* o)
{
    int b = 0;
    while (b < a->B && a->qstart[b + 1] <= r) ++b;
    if (b >= a->B || r < a->qstart[b]) return ORC_EINVAL;
    const int64_t n = a->qstart[b + 1] - a->qstart[b];
    const int64_t pos = (int64_t)a->ctx[b] - n + (r - a->qstart[b]);
    if (pos < 0) return ORC_EINVAL;                  /* more queries than tokens */
    return attend(a, b, r * a->q_sb + (int64_t)h * a->q_sh, pos + 1, h, o);
}

static void* run_slice(void* p)
{
    orc_slice* s = (orc_slice*)p;
    const orc_args* a = s->a;
    s->status = ORC_OK;
    for (int64_t it = s->begin; it < s->end; ++it) {
        int rc;
        if (a->qstart) {
            rc = attend_query(a, it / a->Hq, (int)(it % a->Hq), a->out + it * a->D);
        } else {
            int b, h;
            if (a->pairs) { b = a->pairs[2 * it]; h = a->pairs[2 * it + 1]; }
            else { b = (int)(it / a->Hq); h = (int)(it % a->Hq); }
            if (b < 0 || b >= a->B || h < 0 || h >= a->Hq) { s->status = ORC_EINVAL; return NULL; }
            rc = attend_row(a, b, h, a->out + it * a->D);
        }
        if (rc != ORC_OK) { s->status = rc; return NULL; }
    }
    return NULL;
}

static int run(orc_args* a, int n_threads)
{
    if (!a->q || !a->k || !a->v || !a->bt || !a->ctx || !a->out) return ORC_EINVAL;
    if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->D <= 0 || a->P <= 0) return ORC_EINVAL;
    if (a->Hq % a->Hkv != 0) return ORC_EINVAL;
    if (a->n_items == 0) return ORC_OK;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > a->n_items) n_threads = (int)a->n_items;

    orc_slice* sl = (orc_slice*)calloc((size_t)n_threads, sizeof *sl);
    pthread_t* th = (pthread_t*)calloc((size_t)n_threads, sizeof *th);
    if (!sl || !th) { free(sl); free(th); return ORC_ENOMEM; }
    int64_t per = (a->n_items + n_threads - 1) / n_threads;
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        sl[i].a = a;
        sl[i].begin = (int64_t)i * per;
        sl[i].end = sl[i].begin + per < a->n_items ? sl[i].begin + per : a->n_items;
        if (sl[i].begin >= sl[i].end) continue;
        if (i == n_threads - 1 || pthread_create(&th[i], NULL, run_slice, &sl[i]) != 0) {
            run_slice(&sl[i]);          /* last slice (or a failed spawn) inline */
            sl[i].begin = -1;
        } else {
            ++started;
        }
    }
    int rc = ORC_OK;
    for (int i = 0; i < n_threads; ++i) {
        if (sl[i].begin >= 0 && sl[i].begin < sl[i].end) pthread_join(th[i], NULL);
        if (sl[i].status != ORC_OK && rc == ORC_OK) rc = sl[i].status;
    }
    (void)started;
    free(sl);
    free(th);
    return rc;
}

static void fill(orc_args* a,
                 const void* q, int64_t q_sb, int64_t q_sh,
                 const void* k, const void* v,
                 int64_t s_page, int64_t s_slot, int64_t s_head, int64_t num_pages,
                 const int32_t* bt, int64_t max_blk, const int32_t* ctx,
                 int B, int Hq, int Hkv, int D, int P, float scale)
{
    memset(a, 0, sizeof *a);
    a->q_dtype = ORC_BF16;
    a->kv_dtype = ORC_BF16;
    a->q = q; a->q_sb = q_sb; a->q_sh = q_sh;
    a->k = k; a->v = v;
    a->s_page = s_page; a->s_slot = s_slot; a->s_head = s_head;
    a->num_pages = num_pages;
    a->bt = bt; a->max_blk = max_blk; a->ctx = ctx;
    a->B = B; a->Hq = Hq; a->Hkv = Hkv; a->D = D; a->P = P;
    a->scale = (double)scale;
}

/* Every (b, h) row: out is [B][Hq][D] fp64. */
int pa_oracle_f64(const uint16_t* q, int64_t q_sb, int64_t q_sh,
                  const uint16_t* k, const uint16_t* v,
                  int64_t s_page, int64_t s_slot, int64_t s_head, int64_t num_pages,
                  const int32_t* bt, int64_t max_blk, const int32_t* ctx,
                  int B, int Hq, int Hkv, int D, int P, float scale,
                  double* out, int n_threads)
{
    orc_args a;
    fill(&a, q, q_sb, q_sh, k, v, s_page, s_slot, s_head, num_pages, bt, max_blk, ctx,
         B, Hq, Hkv, D, P, scale);
    a.out = out;
    a.n_items = (int64_t)B * Hq;
    return run(&a, n_threads);
}

/* Selected rows: pairs holds n_pairs (b, h) int32 pairs; out is [n_pairs][D]. */
int pa_oracle_f64_pairs(const uint16_t* q, int64_t q_sb, int64_t q_sh,
                        const uint16_t* k, const uint16_t* v,
                        int64_t s_page, int64_t s_slot, int64_t s_head, int64_t num_pages,
                        const int32_t* bt, int64_t max_blk, const int32_t* ctx,
                        int B, int Hq, int Hkv, int D, int P, float scale,
                        const int32_t* pairs, int64_t n_pairs, double* out, int n_threads)
{
    orc_args a;
    fill(&a, q, q_sb, q_sh, k, v, s_page, s_slot, s_head, num_pages, bt, max_blk, ctx,
         B, Hq, Hkv, D, P, scale);
    a.out = out;
    a.pairs = pairs;
    a.n_items = n_pairs;
    return run(&a, n_threads);
}

/* Every (b, h) row with a sliding window of `window` tokens (0 = none), and
 * an optional planted mistake (0 = none; tests of the pins only). */
int pa_oracle_f64_window(const uint16_t* q, int64_t q_sb, int64_t q_sh,
                         const uint16_t* k, const uint16_t* v,
                         int64_t s_page, int64_t s_slot, int64_t s_head, int64_t num_pages,
                         const int32_t* bt, int64_t max_blk, const int32_t* ctx,
                         int B, int Hq, int Hkv, int D, int P, float scale,
                         int64_t window, double* out, int n_threads, int mutant)
{
    orc_args a;
    if (window < 0) return ORC_EINVAL;
    fill(&a, q, q_sb, q_sh, k, v, s_page, s_slot, s_head, num_pages, bt, max_blk, ctx,
         B, Hq, Hkv, D, P, scale);
    a.out = out;
    a.n_items = (int64_t)B * Hq;
    a.window = window;
    a.mutant = mutant;
    return run(&a, n_threads);
}

/* Every (b, h) row, with element types for Q and for the K/V pools
 * (ORC_BF16 = 1, ORC_F32 = 3, ORC_F16 = 4), a sliding window (0 = none) and
 * an optional planted mistake (0 = none). */
int pa_oracle_f64_typed(const void* q, int64_t q_sb, int64_t q_sh,
                        const void* k, const void* v,
                        int64_t s_page, int64_t s_slot, int64_t s_head, int64_t num_pages,
                        const int32_t* bt, int64_t max_blk, const int32_t* ctx,
                        int B, int Hq, int Hkv, int D, int P, float scale,
                        int q_dtype, int kv_dtype, int64_t window, double* out, int n_threads, int mutant)
{
    orc_args a;
    if (window < 0) return ORC_EINVAL;
    for (int i = 0; i < 2; ++i) {
        int t = i ? kv_dtype : q_dtype;
        if (t != ORC_BF16 && t != ORC_F16 && t != ORC_F32) return ORC_EINVAL;
    }
    fill(&a, q, q_sb, q_sh, k, v, s_page, s_slot, s_head, num_pages, bt, max_blk, ctx,
         B, Hq, Hkv, D, P, scale);
    a.q_dtype = q_dtype;
    a.kv_dtype = kv_dtype;
    a.out = out;
    a.n_items = (int64_t)B * Hq;
    a.window = window;
    a.mutant = mutant;
    return run(&a, n_threads);
}

/* Several queries per sequence: q is [n_rows][Hq][D] with sequence b's
 * queries at rows [qstart[b], qstart[b+1]) (its last tokens); out is
 * [n_rows][Hq][D].  Element types, window and mutant as above. */
int pa_oracle_f64_queries(const void* q, int64_t q_sb, int64_t q_sh,
                          const void* k, const void* v,
                          int64_t s_page, int64_t s_slot, int64_t s_head, int64_t num_pages,
                          const int32_t* bt, int64_t max_blk, const int32_t* ctx,
                          int B, int Hq, int Hkv, int D, int P, float scale,
                          const int32_t* qstart, int64_t n_rows,
                          int q_dtype, int kv_dtype, int64_t window, double* out, int n_threads,
                          int mutant)
{
    orc_args a;
    if (window < 0 || !qstart || n_rows < 0) return ORC_EINVAL;
    if (qstart[0] != 0 || qstart[B] != n_rows) return ORC_EINVAL;
    for (int b = 0; b < B; ++b)
        if (qstart[b + 1] < qstart[b]) return ORC_EINVAL;
    fill(&a, q, q_sb, q_sh, k, v, s_page, s_slot, s_head, num_pages, bt, max_blk, ctx,
         B, Hq, Hkv, D, P, scale);
    a.q_dtype = q_dtype;
    a.kv_dtype = kv_dtype;
    a.qstart = qstart;
    a.n_rows = n_rows;
    a.out = out;
    a.n_items = n_rows * Hq;
    a.window = window;
    a.mutant = mutant;
    return run(&a, n_threads);
}

/* Decodes of one element type over n bit patterns (tests of the decoder). */
int pa_oracle_decode(const void* bits, int dtype, int64_t n, double* out)
{
    if (dtype != ORC_BF16 && dtype != ORC_F16 && dtype != ORC_F32) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = elem(bits, i, dtype);
    return ORC_OK;
}

/* Selected rows with a sliding window (see above). */
int pa_oracle_f64_pairs_window(const uint16_t* q, int64_t q_sb, int64_t q_sh,
                               const uint16_t* k, const uint16_t* v,
                               int64_t s_page, int64_t s_slot, int64_t s_head, int64_t num_pages,
                               const int32_t* bt, int64_t max_blk, const int32_t* ctx,
                               int B, int Hq, int Hkv, int D, int P, float scale,
                               int64_t window, const int32_t* pairs, int64_t n_pairs, double* out,
                               int n_threads)
{
    orc_args a;
    if (window < 0) return ORC_EINVAL;
    fill(&a, q, q_sb, q_sh, k, v, s_page, s_slot, s_head, num_pages, bt, max_blk, ctx,
         B, Hq, Hkv, D, P, scale);
    a.out = out;
    a.pairs = pairs;
    a.n_items = n_pairs;
    a.window = window;
    return run(&a, n_threads);
}

/* As pa_oracle_f64 with a planted mistake (tests of the pins only). */
int pa_oracle_f64_mutant(const uint16_t* q, int64_t q_sb, int64_t q_sh,
                         const uint16_t* k, const uint16_t* v,
                         int64_t s_page, int64_t s_slot, int64_t s_head, int64_t num_pages,
                         const int32_t* bt, int64_t max_blk, const int32_t* ctx,
                         int B, int Hq, int Hkv, int D, int P, float scale,
                         double* out, int n_threads, int mutant)
{
    orc_args a;
    fill(&a, q, q_sb, q_sh, k, v, s_page, s_slot, s_head, num_pages, bt, max_blk, ctx,
         B, Hq, Hkv, D, P, scale);
    a.out = out;
    a.n_items = (int64_t)B * Hq;
    a.mutant = mutant;
    return run(&a, n_threads);
}

int pa_oracle_num_mutants(void) { return 10; }
