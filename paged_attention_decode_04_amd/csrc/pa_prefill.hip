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
    if (!mfma_supported(head_dim, 16, kv_dtype) || 16 % (p.Hq / p.Hkv)) return hipErrorInvalidValue;
    if (kv_dtype == kDtF16)
        return head_dim == 128 ? launch_prefill_d<128, KvF16>(p, split, s) : launch_prefill_d<256, KvF16>(p, split, s);
    return head_dim == 128 ? launch_prefill_d<128, KvBF16>(p, split, s) : launch_prefill_d<256, KvBF16>(p, split, s);
}

}  // namespace pa
