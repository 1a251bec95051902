// pa_prefill.hip -- several queries per sequence (chunked prefill, or a
// batch mixing prefill chunks and decode steps) on the gfx950 matrix cores.
//
// Sequence b's query rows [qstart[b], qstart[b+1]) of q are its last n_b
// tokens: the query at position pos attends causally to [0, pos] (with a
// window W: [pos - W + 1, pos]).  One query per sequence is decode.  (The
// pages name vLLM's chunked-prefill paged-decode path -- page 1, issue
// "ROCm gfx1200: PagedAttnOnline is 8.1x slower per call", section "Where
// to look" -- and owe d=128 prefill -- page 2, "Not claimed".)
//
// A query block is up to 16 / qg consecutive query tokens of one sequence
// times the qg query heads of one KV head: the 16 columns of the MFMA tile
// (column n = token n / qg, head g * qg + n % qg).  The block's K/V tiles
// are read once for all its columns; each column is masked to its own
// causal range, per lane, in the tile step.  Workgroups find their sequence
// on the device: a block prefix sum over the sequences' query counts (in
// LDS) and a binary search.  Long contexts split into partitions merged per
// (query row, head) with the log-sum-exp rule.
#include "pa_mfma_core.h"

namespace pa {

bool prefill_supported(int head_dim, int kv_dtype) {
    return (head_dim == 128 || head_dim == 256 || head_dim == 512) && (kv_dtype == kDtBF16 || kv_dtype == kDtF16);
}

// The staged kernel keeps NB stages of K and V in LDS and every wave's
// accumulators in registers: head_dim 128 and 256.
bool prefill_staged_supported(int head_dim) { return head_dim == 128 || head_dim == 256; }

// Dynamic LDS (page ids of a fill and the B + 1 block prefix sums) the
// per-block kernel can take beside its static wave-merge buffer: at head_dim
// 512 that buffer is 130 KB of the CU's 160 KB.
size_t prefill_dynamic_lds_limit(int head_dim) {
    const size_t merge = sizeof(MergeLds<512>) + 64;      // + the prefix scan's own
    return head_dim == 512 ? (size_t)160 * 1024 - merge : (size_t)64 * 1024;
}

template <int D, bool SPLIT, bool PAGE16, int NBUF, typename KV>
__global__ __launch_bounds__(kMBlock) void pa_prefill_mfma_kernel(DecodeParams p) {
    constexpr int KK = TileFrag<D>::KK;
    constexpr int NO = D / 16;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int qg = p.Hq / p.Hkv;
    const int qt = 16 / qg;                     // query tokens per block
    const int slot = blockIdx.x % p.n_slots;
    const int rest = blockIdx.x / p.n_slots;
    const int g = rest % p.Hkv;
    const int part = rest / p.Hkv;

    extern __shared__ int s_dyn[];
    int* s_pages = s_dyn;                       // kLeanTokensPerFill / P + 2 entries
    int* s_pref = s_dyn + p.lean_page_slots;    // B + 1 block prefix sums
    block_prefix(p.B, s_pref, [&](int bb) {
        const int nq = max(p.qstart[bb + 1] - p.qstart[bb], 0);
        return (nq + qt - 1) / qt;
    });
    auto sp = [&](int i) { return __builtin_amdgcn_readfirstlane(s_pref[i]); };
    if (slot >= sp(p.B)) return;                // a spare slot of the grid's upper bound
    int lo_b = 0, hi_b = p.B - 1;               // the last sequence with S[b] <= slot
    while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if (sp(mid) <= slot) lo_b = mid; else hi_b = mid - 1;
    }
    const int b = lo_b;
    const int blk = slot - sp(b);
    const int r0 = p.qstart[b];
    const int nq = p.qstart[b + 1] - r0;
    const int tok0 = blk * qt;
    // Rows outside q (a query_start that breaks its precondition) are never
    // touched.
    if (r0 < 0 || r0 + tok0 >= p.q_rows) return;
    const int ntok = min(min(qt, nq - tok0), p.q_rows - (r0 + tok0));
    const int L = clampi(p.ctx[b], 0, p.max_blk * p.P);
    const int pos0 = L - nq + tok0;             // position of the block's first query

    // Column n: query token tok0 + n / qg, head g * qg + n % qg; its tokens
    // [mask_lo, mask_hi).  A position below 0 (more queries than tokens) has
    // no tokens and yields zeros.
    const bool col_live = n < ntok * qg;
    const int pos_n = pos0 + (col_live ? n / qg : 0);
    const int mask_hi = col_live ? pos_n + 1 : 0;
    const int mask_lo = p.window > 0 ? max(0, pos_n - p.window + 1) : 0;
    const int pos_max = pos0 + ntok - 1;
    const int lo_min = p.window > 0 ? max(0, pos0 - p.window + 1) : 0;
    // This partition's tokens: [base + part * T, base + (part + 1) * T) up to
    // the block's last query, where base is the tile holding the block's
    // first attended token (0 without a window).
    const int base = lo_min & ~(kTile - 1);
    const int ts = base + part * p.part_tokens;
    const int te = min(pos_max + 1, ts + p.part_tokens);
    if (SPLIT && ts >= te) return;              // no token here: the merge never reads it

    u32x4 qop[KK];
    {
        const int r = r0 + tok0 + (col_live ? n / qg : 0);
        const int h = g * qg + n % qg;
        const int64_t qr = (int64_t)r * p.q_sb + (int64_t)h * p.q_sh;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int64_t off = qr + k_col<D, false>(kk, n, q);
            u32x4 w;
            if (p.q_dtype == KV::code) {
                w = load16(static_cast<const uint16_t*>(p.q) + off);
            } else {
                float f[8];
                load8f(p.q, p.q_dtype, off, f);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = KV::pack2(f[2 * i], f[2 * i + 1]);
            }
            qop[kk] = col_live ? w : u32x4{0u, 0u, 0u, 0u};
        }
    }

    f32x4 o[NO];
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kEmptyMax, l_run = 0.f;
    LaneOffsets lo;
    lo.k = k_row<D, false>(0, n) * (int)p.k_ss + k_col<D, false>(0, n, q);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) lo.v[jj] = (4 * q + jj) * (int)p.v_ss + 8 * n;
    for (int c0 = ts; c0 < te; c0 += kLeanTokensPerFill) {
        const int c1 = min(te, c0 + kLeanTokensPerFill);
        int pg0, lp1, unused;
        page_slot(p, c0, pg0, unused);
        page_slot(p, c1 - 1, lp1, unused);
        if (c0 != ts) __syncthreads();          // the previous chunk's page ids are in use until here
        fetch_pages(p, b, pg0, lp1, s_pages, tid);
        __syncthreads();
        run_tiles<D, PAGE16, false, NBUF, KV>(p, s_pages, pg0, g, n, q, wave, lo, qop, col_live, c0, c1, lo_min,
                                              mask_lo, mask_hi, o, m_run, l_run);
    }
    l_run = xsum32(xsum16(l_run));

    __shared__ MergeLds<D> lds;
    merge_waves<D>(lds, o, m_run, l_run, ntok * qg, n, q, wave, tid,
                   [&](int jq, int d0, const float (&ov)[8], float lse) {
        const int64_t r = r0 + tok0 + jq / qg;
        const int h = g * qg + jq % qg;
        if constexpr (!SPLIT) {
            store8(p.out, p.out_dtype, r * p.o_sb + (int64_t)h * p.o_sh + d0, ov);
        } else {
            const int64_t s = (r * p.Hq + h) * p.n_part + part;
            store_f32x8(p.part_o + s * D + d0, ov);
            if (d0 == 0) p.part_lse[s] = lse;
        }
    });
}

// Merge of the partitions of query row r, head h: the partitions its causal
// (and window) range meets, first to last.
template <int D>
__global__ __launch_bounds__(64) void pa_prefill_merge_kernel(DecodeParams p) {
    const int h = blockIdx.x, r = blockIdx.y;
    int lo_b = 0, hi_b = p.B - 1;               // the last sequence with qstart[b] <= r
    while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if (p.qstart[mid] <= r) lo_b = mid; else hi_b = mid - 1;
    }
    const int b = lo_b;
    const int nq = p.qstart[b + 1] - p.qstart[b];
    const int L = clampi(p.ctx[b], 0, p.max_blk * p.P);
    const int i = r - p.qstart[b];              // query index inside the sequence
    const int pos = L - nq + i;
    int first = 0, count = 0;
    if (pos >= 0) {
        // the partitions are relative to the base of the row's query block
        const int qt = 16 / (p.Hq / p.Hkv);
        const int pos0 = L - nq + (i / qt) * qt;
        const int base = (p.window > 0 ? max(0, pos0 - p.window + 1) : 0) & ~(kTile - 1);
        const int lo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
        first = (lo - base) / p.part_tokens;
        count = (pos - base) / p.part_tokens - first + 1;
    }
    merge_partials<D>(p, ((int64_t)r * p.Hq + h) * p.n_part + first, 1, count,
                      (int64_t)r * p.o_sb + (int64_t)h * p.o_sh);
}

// ---------------------------------------------------------------------------
// Staged layout, for calls with many query blocks: a workgroup of NW waves
// takes NW consecutive query blocks of one sequence (one per wave) and one
// KV head.  K and V stream through LDS in stages of ST tokens, read from
// memory once per workgroup and consumed by every wave; each wave keeps its
// own columns' online-softmax state over the whole range, so there is
// neither a split nor a wave merge.
//
// The stages arrive by direct global-to-LDS loads (no registers on the way),
// NB - 1 stages ahead of the one being consumed, into NB rotating buffers.
// LDS rows are D elements with no padding; the 16-byte chunk c of row r sits
// at chunk position c ^ f(r & 15): f moves row bits 0, 1, 2 to bits 3, 2, 1
// and maps row bit 3 to 3 (0b0011).  Each half-wave of a transposing V read
// takes 2 chunks of 8 consecutive rows (LDS serves 32 lanes of such a read
// per cycle from 64 four-byte banks): f sends those rows to 8 distinct
// values of chunk bits 1..3, so the 16 chunks read are distinct and hit
// every bank once; a plain XOR with the row would use 8 chunks twice (a
// 2-way conflict).  The K reads (16 rows, one chunk each) stay conflict-free
// with this f as with the XOR, where a plain rotation of the row bits would
// not (both measured with LDS counters).
template <int D, int NW, int NB>
struct Staged {
    static constexpr int NT = NW * 64;
    static constexpr int ST = D == 128 ? 64 : 32;    // tokens per stage (whole 32-token pairs)
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int BLK = ST * CPR / 64;        // 1 KiB blocks per tensor and stage
    static constexpr int LPW = BLK / NW;             // blocks per wave per tensor and stage
    static constexpr int STAGE = ST * D;             // elements per tensor and stage
    static constexpr int kFillTokens = 2048;         // tokens per page-id fill
    static_assert(BLK % NW == 0 && ST % 32 == 0, "stage must split evenly over the waves");
    static_assert(2 * LPW * (NB - 2) <= 63, "outstanding loads must fit the vector-memory counter");
};

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_tr(const uint16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(__attribute__((address_space(3))) void*)(p)));
}
// Element offset, inside its row, of chunk `chunk` of row `row`.
__device__ __forceinline__ int swz_row(int row) {
    return (((row & 1) << 3) | ((row & 2) << 1) | ((row & 4) >> 1)) ^ (((row >> 3) & 1) * 3);
}
__device__ __forceinline__ int swz(int row, int chunk) { return (chunk ^ swz_row(row)) << 3; }

// Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS operations are done, then meet the workgroup.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// 32 tokens tb .. tb + 31 from one stage buffer (rows 0 .. 31 of kl / vl),
// in two steps so that a stage can issue the logits of all its pairs before
// the first softmax (the matrix cores then overlap the vector work):
// stage_logits: the logits of the two 16-token halves of each pair on MFMA;
// pair_update: one online-softmax update, and P.V as one 16x16x32 MFMA per
// 16 dims whose contraction runs over both halves (lane q's eight k-slots:
// tokens 4q .. 4q+3 of each half).  P enters P.V as the sum of two KV-type
// values, hi = round(p) and lo = round(p - hi): the weights are then exact to
// about 2^-17 relative, and the normaliser sums those same weights.
//
// Products into one accumulator are spaced apart: with accumulators in
// VGPRs, an MFMA that reads the previous one's result waits for it (a chain
// of dependent 16x16x32 MFMAs runs at about a third of the issue rate).
// The logits of all NPAIR pairs are accumulated k-step by k-step, 2 NPAIR
// chains side by side.
template <int D, int NPAIR, typename KV>
__device__ __forceinline__ void stage_logits(const uint16_t* kl, const u32x4 (&qop)[D / 32], int n, int q,
                                             f32x4 (&sa)[NPAIR], f32x4 (&sb)[NPAIR]) {
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
        sa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        sb[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int i = 0; i < NPAIR; ++i) {
            const uint16_t* kli = kl + 32 * i * D;
            sa[i] = KV::mma_qk(lds16(kli + n * D + swz(n, 4 * kk + q)), qop[kk], sa[i]);
            sb[i] = KV::mma_qk(lds16(kli + (16 + n) * D + swz(16 + n, 4 * kk + q)), qop[kk], sb[i]);
        }
}

// Raise this wave's issue priority over a block of matrix-core work and
// drop it after: while some waves of the CU run their softmax, the ones with
// MFMAs ready keep the matrix pipe fed.  Measured on chunked prefill: 2.5%
// faster at head_dim 128 (four waves per SIMD), 5% slower at 256 (two), so
// only head_dim 128 uses it.  sched_barrier keeps the compiler from moving
// work across the switch.
template <int D, int LEVEL>
__device__ __forceinline__ void mfma_prio() {
    if constexpr (D == 128) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(LEVEL);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The online-softmax update of one 32-token pair from its logits (sa: tokens
// tb + 4q + r, sb: the same + 16, for lane column n): the reference max and
// the accumulators move when needed, and the pair's weights come back as the
// two bf16/fp16 parts of P^T, hi = round(p) and lo = round(p - hi).
template <int D, typename KV>
__device__ __forceinline__ void pair_softmax(const DecodeParams& p, const f32x4& sa, const f32x4& sb, int tb,
                                             bool mask, int mask_lo, int mask_hi, int q, bool col_live,
                                             f32x4 (&o)[D / 16], float& m_run, f32x4& l_acc, u32x4& ph,
                                             u32x4& pl) {
    constexpr int NO = D / 16;
    const float sc = p.scale_log2;
    auto live = [&](int t) { return col_live && t < mask_hi && t >= mask_lo; };
    // Exponents relative to the reference max, one fma each; the column max
    // is only formed when some logit passes the reference by more than
    // kRescaleSlack (then, as in tile_step, the reference moves and the
    // accumulators rescale).
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        x[r] = fmaf(sa[r], sc, -m_run);
        x[4 + r] = fmaf(sb[r], sc, -m_run);
    }
    if (mask) {                                 // (wave-uniform) else every token is in every column's range
        const int t0 = tb + 4 * q;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x[r] = live(t0 + r) ? x[r] : -INFINITY;
            x[4 + r] = live(t0 + 16 + r) ? x[4 + r] : -INFINITY;
        }
    }
    const float xm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    if (__any(xm > kRescaleSlack)) {
        float sv[8];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tb + 4 * q + r;
            sv[r] = sa[r] * sc;
            sv[4 + r] = sb[r] * sc;
            if (mask) {
                sv[r] = live(t) ? sv[r] : -INFINITY;
                sv[4 + r] = live(t + 16) ? sv[4 + r] : -INFINITY;
            }
            mt = fmaxf(mt, fmaxf(sv[r], sv[4 + r]));
        }
        mt = xmax32(xmax16(mt));
        const float mn = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - mn);
        m_run = mn;
        l_acc *= alpha;
#pragma unroll
        for (int i = 0; i < NO; ++i) o[i] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = sv[i] - mn;
    }
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(x[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ph[i] = KV::pack2(pr[2 * i], pr[2 * i + 1]);
        pl[i] = KV::pack2(pr[2 * i] - KV::lo(ph[i]), pr[2 * i + 1] - KV::hi(ph[i]));
    }
}

// The normaliser on the matrix cores: an all-ones operand times P^T sums
// each column's weights (hi + lo, exactly the ones P.V uses) over all 32
// tokens, in every row of the tile.
template <typename KV>
__device__ __forceinline__ u32x4 ones_operand() {
    const uint32_t one2 = KV::pack2(1.f, 1.f);
    return u32x4{one2, one2, one2, one2};
}

// P.V output tiles taken G at a time: the G hi products, then the G lo
// products, so that the two products into one accumulator are G MFMAs
// apart.  4 at head_dim 256; 2 at 128, where 4 would take the kernel past
// 128 VGPRs and cost the second workgroup per CU.
template <int D>
constexpr int kPvGroup = D == 128 ? 2 : 4;

// V^T operands by transposing LDS reads (ds_read_b64_tr_b16): inside each
// 16-lane group, lane j gets slot k from element j % 4 of the 8 bytes at
// the address of lane 4k + j / 4.  Lane 4k + m of group q points at V row
// 4q + k, dims 16t + 4m .. +3, so lane (j, q) receives tokens 4q .. 4q+3
// of dim 16t + j: the A operand of output tile t (rows = dims 16t ..
// 16t + 15), one read per half.  Rows are swizzled like the K reads.
template <int D>
__device__ __forceinline__ u32x4 v_operand(const uint16_t* vl, int n, int q, int t) {
    const int vx = 4 * q + (n >> 2);            // row inside the half (= row & 15)
    const int vy = ((n >> 1) & 1) ^ swz_row(vx);
    const int off = vx * D + 4 * (n & 1) + (((2 * t) ^ vy) << 3);
    const u32x2 a = lds_tr(vl + off), b = lds_tr(vl + 16 * D + off);
    return u32x4{a[0], a[1], b[0], b[1]};
}

template <int D, typename KV>
__device__ __forceinline__ void pair_update(const DecodeParams& p, const uint16_t* vl, const f32x4& sa,
                                            const f32x4& sb, int tb, bool mask, int mask_lo, int mask_hi, int n,
                                            int q, bool col_live, f32x4 (&o)[D / 16], float& m_run, f32x4& l_acc) {
    constexpr int NO = D / 16;
    constexpr int G = kPvGroup<D>;
    static_assert(NO % G == 0, "P.V groups");
    u32x4 ph, pl;
    pair_softmax<D, KV>(p, sa, sb, tb, mask, mask_lo, mask_hi, q, col_live, o, m_run, l_acc, ph, pl);
    mfma_prio<D, 1>();
    const u32x4 ones = ones_operand<KV>();
    l_acc = KV::mma_qk(ones, ph, l_acc);        // the normaliser's lo product comes after the P.V ones
#pragma unroll
    for (int t0 = 0; t0 < NO; t0 += G) {
        u32x4 vt[G];
#pragma unroll
        for (int j = 0; j < G; ++j) vt[j] = v_operand<D>(vl, n, q, t0 + j);
#pragma unroll
        for (int j = 0; j < G; ++j) o[t0 + j] = KV::mma_qk(vt[j], ph, o[t0 + j]);
#pragma unroll
        for (int j = 0; j < G; ++j) o[t0 + j] = KV::mma_qk(vt[j], pl, o[t0 + j]);
    }
    l_acc = KV::mma_qk(ones, pl, l_acc);
    mfma_prio<D, 0>();
}

// Per-lane byte offsets of this lane's 16-byte chunk inside a block of
// consecutive K (V) rows that starts at a given slot of one page: row
// lane / CPR of the block, the chunk that the swizzle puts at position
// lane % CPR.  A block's rows 0 .. 15 position is the same for every block
// this wave loads (static_assert in the kernel), so one pair serves all.
struct IssueLane {
    uint32_t k, v;
};

// This wave's share of stage s of the fill starting at token c0: blocks
// j * NW + wave of K and of V, by direct global-to-LDS loads.  Rows are
// clamped into [lo_min, te), which lies in this fill's pages.  When no row of
// the stage is clamped and every block's rows share a page (the page size a
// multiple of the rows per block), each block's page and first slot are
// wave-uniform: the address is a scalar base plus the lane's fixed offset.
template <int D, int NW, int NB>
__device__ __forceinline__ void staged_issue(const DecodeParams& p, const uint16_t* __restrict__ kb,
                                             const uint16_t* __restrict__ vb, const int* __restrict__ s_pages,
                                             uint16_t* __restrict__ kd, uint16_t* __restrict__ vd, int c0, int s,
                                             int pg0, int lo_min, int te, int wave, int lane, bool blk_in_page,
                                             const IssueLane& il) {
    using C = Staged<D, NW, NB>;
    constexpr int RPB = 64 / C::CPR;            // rows per 1 KiB block
    const int r0 = c0 + s * C::ST;
    if (blk_in_page && r0 >= lo_min && r0 + C::ST <= te) {             // wave-uniform
        int page[C::LPW], sl[C::LPW];
#pragma unroll
        for (int j = 0; j < C::LPW; ++j) {
            int lp;
            page_slot(p, r0 + (j * NW + wave) * RPB, lp, sl[j]);
            page[j] = s_pages[lp - pg0];
        }
#pragma unroll
        for (int j = 0; j < C::LPW; ++j) {
            const int cb = j * NW + wave;
            const uint32_t pg = (uint32_t)__builtin_amdgcn_readfirstlane(page[j]);
            const uint32_t slu = (uint32_t)__builtin_amdgcn_readfirstlane(sl[j]);
            // 32-bit page stride, 24-bit slot stride (the host checks both)
            const char* ks = reinterpret_cast<const char*>(kb) + 2 * ((uint64_t)pg * (uint32_t)p.k_sp + slu * (uint32_t)p.k_ss);
            const char* vs = reinterpret_cast<const char*>(vb) + 2 * ((uint64_t)pg * (uint32_t)p.v_sp + slu * (uint32_t)p.v_ss);
            __builtin_amdgcn_global_load_lds(ks + il.k, kd + cb * 512, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vs + il.v, vd + cb * 512, 16, 0, 0);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
        const int cb = j * NW + wave;
        const int lin = cb * 64 + lane;
        const int row = lin / C::CPR;
        const int chunk = (lin % C::CPR) ^ swz_row(row);
        const int t = clampi(r0 + row, lo_min, te - 1);
        int lp, sl;
        page_slot(p, t, lp, sl);
        const uint32_t page = (uint32_t)s_pages[lp - pg0];
        const uint64_t ko = (uint64_t)page * (uint32_t)p.k_sp + (uint32_t)(__mul24(sl, (int)p.k_ss) + chunk * 8);
        const uint64_t vo = (uint64_t)page * (uint32_t)p.v_sp + (uint32_t)(__mul24(sl, (int)p.v_ss) + chunk * 8);
        __builtin_amdgcn_global_load_lds(kb + ko, kd + cb * 512, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + vo, vd + cb * 512, 16, 0, 0);
    }
}

// One stage: issue stage st + NB - 1 into the free buffer (kd, vd) when
// do_issue, then consume stage st from (kl, vl).  The two buffer pairs are
// distinct (restrict): the compiler then knows that the stage reads do not
// depend on the loads just issued and adds no wait for them; the wait for
// stage st itself is the explicit one before the call.
template <int D, int NW, int NB, typename KV>
__device__ __forceinline__ void staged_stage(const DecodeParams& p, const uint16_t* __restrict__ kb,
                                             const uint16_t* __restrict__ vb, const int* __restrict__ s_pages,
                                             uint16_t* __restrict__ kd, uint16_t* __restrict__ vd, bool do_issue,
                                             const uint16_t* __restrict__ kl, const uint16_t* __restrict__ vl,
                                             int c0, int st, int pg0, int lo_min, int te, int wave, int lane,
                                             bool blk_in_page, const IssueLane& il, int ntok,
                                             const u32x4 (&qop)[D / 32], int n, int q, int free_lo, int free_hi,
                                             int mask_lo, int mask_hi, bool col_live, f32x4 (&o)[D / 16],
                                             float& m_run, f32x4& l_acc) {
    using C = Staged<D, NW, NB>;
    if (do_issue)
        staged_issue<D, NW, NB>(p, kb, vb, s_pages, kd, vd, c0, st + NB - 1, pg0, lo_min, te, wave, lane, blk_in_page,
                                il);
    // A wave with no query (the last workgroup of a sequence, or few queries
    // per sequence) only loads its share of every stage.
    if (ntok == 0) return;                                          // wave-uniform
    const int sb0 = c0 + st * C::ST;
    constexpr int NPAIR = C::ST / 32;
    f32x4 sa[NPAIR], sb[NPAIR];
    mfma_prio<D, 1>();
    stage_logits<D, NPAIR, KV>(kl, qop, n, q, sa, sb);
    mfma_prio<D, 0>();
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
        const int tb = sb0 + 32 * i;
        const bool mask = !(tb >= free_lo && tb + 32 <= free_hi);   // wave-uniform
        pair_update<D, KV>(p, vl + 32 * i * D, sa[i], sb[i], tb, mask, mask_lo, mask_hi, n, q, col_live, o, m_run,
                           l_acc);
    }
}

template <int D, int NW, int NB, typename KV>
__global__ __launch_bounds__(NW * 64) void pa_prefill_staged_kernel(DecodeParams p) {
    using C = Staged<D, NW, NB>;
    constexpr int KK = D / 32;
    constexpr int NO = D / 16;
    constexpr int NT = C::NT, ST = C::ST, LPW = C::LPW;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int qg = p.Hq / p.Hkv;
    const int qt = 16 / qg;                     // query tokens per block
    const int gq = NW * qt;                     // query tokens per workgroup
    // Workgroups go round-robin over the 8 dies (XCDs), each with its own L2:
    // renumber so that each die runs a contiguous range of (KV head, slot),
    // whose neighbours read the same sequence's K/V.
    const int nwg = gridDim.x, xcd = blockIdx.x & 7, per = nwg >> 3, rem = nwg & 7;
    const int lid = xcd * per + min(xcd, rem) + (blockIdx.x >> 3);
    const int slot = lid % p.n_slots;
    const int g = lid / p.n_slots;

    extern __shared__ int s_dyn[];
    int* s_pages = s_dyn;                       // kFillTokens / P + 2 entries
    int* s_pref = s_dyn + p.lean_page_slots;    // B + 1 prefix sums of workgroup slots
    block_prefix<NT>(p.B, s_pref, [&](int bb) {
        const int nq = max(p.qstart[bb + 1] - p.qstart[bb], 0);
        return (nq + gq - 1) / gq;
    });
    auto sp = [&](int i) { return __builtin_amdgcn_readfirstlane(s_pref[i]); };
    if (slot >= sp(p.B)) return;
    int lo_b = 0, hi_b = p.B - 1;
    while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if (sp(mid) <= slot) lo_b = mid; else hi_b = mid - 1;
    }
    const int b = lo_b;
    const int r0 = p.qstart[b];
    const int nq = p.qstart[b + 1] - r0;
    const int gtok0 = (slot - sp(b)) * gq;      // the workgroup's first query token
    if (r0 < 0 || r0 + gtok0 >= p.q_rows) return;
    const int gntok = min(min(gq, nq - gtok0), p.q_rows - (r0 + gtok0));
    const int Lb = clampi(p.ctx[b], 0, p.max_blk * p.P);

    // This wave's block: query tokens tok0 .. tok0 + ntok - 1 of the sequence.
    const int tok0 = gtok0 + wave * qt;
    const int ntok = clampi(gntok - wave * qt, 0, qt);
    const bool col_live = n < ntok * qg;
    const int pos_n = Lb - nq + tok0 + (col_live ? n / qg : 0);
    const int mask_hi = col_live ? pos_n + 1 : 0;
    const int mask_lo = p.window > 0 ? max(0, pos_n - p.window + 1) : 0;
    // Tokens [free_lo, free_hi) lie in every column's range (none if a
    // column is empty): pairs inside it skip the masking.
    const bool full = ntok == qt;
    const int free_hi = full ? Lb - nq + tok0 + 1 : INT32_MIN;
    const int free_lo = p.window > 0 ? max(0, Lb - nq + tok0 + qt - p.window) : 0;
    // The workgroup's tokens: from its first query's window start (a tile
    // boundary below it) to its last query.
    const int pos_first = Lb - nq + gtok0;
    const int te = pos_first + gntok;
    const int lo_min = p.window > 0 ? max(0, pos_first - p.window + 1) : 0;
    const int ts = lo_min & ~(kTile - 1);

    u32x4 qop[KK];
    {
        const int r = r0 + tok0 + (col_live ? n / qg : 0);
        const int h = g * qg + n % qg;
        const int64_t qr = (int64_t)r * p.q_sb + (int64_t)h * p.q_sh;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int64_t off = qr + 32 * kk + 8 * q;
            u32x4 w = u32x4{0u, 0u, 0u, 0u};
            if (col_live) {
                if (p.q_dtype == KV::code) {
                    w = load16(static_cast<const uint16_t*>(p.q) + off);
                } else {
                    float f[8];
                    load8f(p.q, p.q_dtype, off, f);
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = KV::pack2(f[2 * i], f[2 * i + 1]);
                }
            }
            qop[kk] = w;
        }
    }

    f32x4 o[NO];
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kEmptyMax;
    f32x4 l_acc = {0.f, 0.f, 0.f, 0.f};         // every element: the lane's column sum of weights
    __shared__ __attribute__((aligned(16))) uint16_t s_kv[NB][2][C::STAGE];
    const uint16_t* kb = static_cast<const uint16_t*>(p.k) + (int64_t)g * p.k_sh;
    const uint16_t* vb = static_cast<const uint16_t*>(p.v) + (int64_t)g * p.v_sh;

    constexpr int RPB = 64 / C::CPR;            // rows per 1 KiB block of a stage
    static_assert((NW * RPB) % 16 == 0, "a lane's swizzle row must be the same in every block it loads");
    const bool blk_in_page = p.P % RPB == 0;
    IssueLane il;
    {
        const int row = wave * RPB + lane / C::CPR;                  // mod 16, the same for every block
        const uint32_t chunk = (uint32_t)((lane % C::CPR) ^ swz_row(row));
        il.k = 2u * ((uint32_t)(lane / C::CPR) * (uint32_t)p.k_ss + chunk * 8u);
        il.v = 2u * ((uint32_t)(lane / C::CPR) * (uint32_t)p.v_ss + chunk * 8u);
    }
    for (int c0 = ts; c0 < te; c0 += C::kFillTokens) {
        const int c1 = min(te, c0 + C::kFillTokens);
        int pg0, lp1, unused;
        page_slot(p, c0, pg0, unused);
        page_slot(p, c1 - 1, lp1, unused);
        fetch_pages<NT>(p, b, pg0, lp1, s_pages, tid);
        __syncthreads();                        // page ids ready; every wave is done with the last chunk
        const int n_st = (c1 - c0 + ST - 1) / ST;
#pragma unroll
        for (int s = 0; s < NB - 1; ++s)
            if (s < n_st)
                staged_issue<D, NW, NB>(p, kb, vb, s_pages, &s_kv[s][0][0], &s_kv[s][1][0], c0, s, pg0, lo_min, te,
                                        wave, lane, blk_in_page, il);
        for (int st = 0; st < n_st; ++st) {
            // Stage st has landed once at most `ahead` later stages are in flight.
            const int ahead = min(NB - 2, n_st - 1 - st);
            if (NB >= 4 && ahead >= 2) vm_wait_barrier<4 * LPW>();
            else if (NB >= 3 && ahead == 1) vm_wait_barrier<2 * LPW>();
            else vm_wait_barrier<0>();
            // The buffer of stage st - 1 is free: every wave has passed the barrier.
            const int nx = (st + NB - 1) % NB, cu = st % NB;
            staged_stage<D, NW, NB, KV>(p, kb, vb, s_pages, &s_kv[nx][0][0], &s_kv[nx][1][0], st + NB - 1 < n_st,
                                        &s_kv[cu][0][0], &s_kv[cu][1][0], c0, st, pg0, lo_min, te, wave, lane,
                                        blk_in_page, il, ntok, qop, n, q, free_lo, free_hi, mask_lo, mask_hi, col_live, o, m_run,
                                        l_acc);
        }
        __syncthreads();                        // every wave is done reading the stage buffers and page ids
    }

    // Each wave holds all tokens of its columns: normalise and store.
    const float inv = l_acc[0] > 0.f ? 1.f / l_acc[0] : 0.f;
    if (col_live) {                             // o[t][r]: dim 16t + 4q + r
        const int64_t r = r0 + tok0 + n / qg;
        const int h = g * qg + n % qg;
        const int64_t base = r * p.o_sb + (int64_t)h * p.o_sh + 4 * q;
#pragma unroll
        for (int t = 0; t < NO; ++t) {
            store2(p.out, p.out_dtype, base + 16 * t, o[t][0] * inv, o[t][1] * inv);
            store2(p.out, p.out_dtype, base + 16 * t + 2, o[t][2] * inv, o[t][3] * inv);
        }
    }
}

// LDS of the staged kernel beyond its dynamic part (page ids of one fill and
// the B + 1 prefix sums of workgroup slots): the K/V stages, and a margin for
// the few scalars the kernel shares (36 bytes now).  pa_prefill takes at most
// 4096 sequences, so even pages of one token leave the whole within the CU's
// 160 KB at both head dims.
template <int D, int NW, int NB>
constexpr size_t staged_static_lds() {
    return sizeof(uint16_t) * NB * 2 * Staged<D, NW, NB>::STAGE + 1024;
}
template <int D, int NW, int NB>
constexpr size_t staged_dynamic_lds(int page_size, int batch) {
    return sizeof(int) * ((size_t)(Staged<D, NW, NB>::kFillTokens / page_size) + 2 + (size_t)batch + 1);
}
constexpr size_t kCuLdsBytes = 160 * 1024;
static_assert(staged_static_lds<128, kStagedWaves, kStagedBuffers128>() +
                  staged_dynamic_lds<128, kStagedWaves, kStagedBuffers128>(1, 4096) <= kCuLdsBytes,
              "staged kernel LDS at head_dim 128");
static_assert(staged_static_lds<256, kStagedWaves, kStagedBuffers256>() +
                  staged_dynamic_lds<256, kStagedWaves, kStagedBuffers256>(1, 4096) <= kCuLdsBytes,
              "staged kernel LDS at head_dim 256");

template <int D, int NW, int NB, typename KV>
static hipError_t launch_staged_d(DecodeParams p, hipStream_t s) {
    using C = Staged<D, NW, NB>;
    p.lean_page_slots = C::kFillTokens / p.P + 2;
    const size_t lds = sizeof(int) * (size_t)(p.lean_page_slots + p.B + 1);
    if (staged_static_lds<D, NW, NB>() + lds > kCuLdsBytes) return hipErrorInvalidValue;
    dim3 grid((uint32_t)((int64_t)p.n_slots * p.Hkv));
    hipLaunchKernelGGL((pa_prefill_staged_kernel<D, NW, NB, KV>), grid, dim3(C::NT), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_prefill_staged(const DecodeParams& p, int head_dim, int kv_dtype, hipStream_t s) {
    if (!prefill_supported(head_dim, kv_dtype) || !prefill_staged_supported(head_dim) || 16 % (p.Hq / p.Hkv))
        return hipErrorInvalidValue;
    constexpr int NW = kStagedWaves, NB1 = kStagedBuffers128, NB2 = kStagedBuffers256;
    if (kv_dtype == kDtF16)
        return head_dim == 128 ? launch_staged_d<128, NW, NB1, KvF16>(p, s) : launch_staged_d<256, NW, NB2, KvF16>(p, s);
    return head_dim == 128 ? launch_staged_d<128, NW, NB1, KvBF16>(p, s) : launch_staged_d<256, NW, NB2, KvBF16>(p, s);
}

template <int D, bool SPLIT, bool PAGE16, typename KV>
static hipError_t launch_prefill_t(const DecodeParams& p, hipStream_t s) {
    constexpr int NBUF = D == 128 ? 3 : 2;
    const size_t lds = sizeof(int) * (size_t)(p.lean_page_slots + p.B + 1);
    dim3 grid((uint32_t)((int64_t)p.n_slots * p.Hkv * p.n_part));
    hipLaunchKernelGGL((pa_prefill_mfma_kernel<D, SPLIT, PAGE16, NBUF, KV>), grid, dim3(kMBlock), lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !SPLIT) return e;
    hipLaunchKernelGGL(pa_prefill_merge_kernel<D>, dim3(p.Hq, p.q_rows), dim3(64), 0, s, p);
    return hipGetLastError();
}

template <int D, typename KV>
static hipError_t launch_prefill_d(const DecodeParams& p, bool split, hipStream_t s) {
    const bool page16 = p.p_shift >= 4 && (int64_t)p.P * (p.k_ss > p.v_ss ? p.k_ss : p.v_ss) < (1ll << 30);
    if (split) return page16 ? launch_prefill_t<D, true, true, KV>(p, s) : launch_prefill_t<D, true, false, KV>(p, s);
    return page16 ? launch_prefill_t<D, false, true, KV>(p, s) : launch_prefill_t<D, false, false, KV>(p, s);
}

hipError_t launch_prefill(const DecodeParams& p, int head_dim, int kv_dtype, bool split, hipStream_t s) {
    if (!prefill_supported(head_dim, kv_dtype) || 16 % (p.Hq / p.Hkv)) return hipErrorInvalidValue;
    if (sizeof(int) * (size_t)(p.lean_page_slots + p.B + 1) > prefill_dynamic_lds_limit(head_dim))
        return hipErrorInvalidValue;
    if (head_dim == 512)
        return kv_dtype == kDtF16 ? launch_prefill_d<512, KvF16>(p, split, s) : launch_prefill_d<512, KvBF16>(p, split, s);
    if (kv_dtype == kDtF16)
        return head_dim == 128 ? launch_prefill_d<128, KvF16>(p, split, s) : launch_prefill_d<256, KvF16>(p, split, s);
    return head_dim == 128 ? launch_prefill_d<128, KvBF16>(p, split, s) : launch_prefill_d<256, KvBF16>(p, split, s);
}

}  // namespace pa
