// pa_mfma.hip -- matrix-core decode paged-attention kernel for gfx950.
//
// One workgroup (4 waves) handles one sequence, the (up to 16) query heads
// of one KV head, and one partition of the tokens.  Each wave walks 16-token
// tiles of the partition (tile j goes to wave j mod 4) and keeps its own
// online-softmax state.  Per tile:
//
//   Logits on v_mfma_f32_16x16x32_bf16, with K rows going straight from
//   global memory into the A operand and Q (bf16, unscaled) as the B operand,
//   loaded once.  Two row layouts:
//   * qg <= 8 ("split" layout): the 16 MFMA rows are 8 tokens x 2 halves of
//     each 64-dim block and the 16 B columns are 8 queries x the same 2
//     halves, so 8 lanes read one whole 128-byte line of a K row per load (8
//     full lines per instruction).  The diagonal (half, half) blocks of the C
//     tile are the two partial dot products; a permlane32 swap plus a DPP
//     row rotate by 8 adds them, and a second swap deals the 16 tokens of
//     two such tiles out so lane l holds query l%16, tokens 4 (l/16) + r.
//   * qg 9..16: row = token, column = query, 16 rows x 64 bytes per load.
//   O^T (D x 16) += V^T_tile (D x 16 tokens) . P^T (16 x 16)
//       v_mfma_f32_16x16x16_bf16, D/16 steps.  P^T is exactly the C tile
//       held as bf16 (lane l: query l%16, tokens 4 (l/16) + jj).  V^T: lane l
//       loads the 16-byte chunk l%16 of the four rows 4 (l/16) + jj (whole
//       256-byte rows per 16 lanes) and transposes the 4 x 8 bf16 block in
//       registers, so MFMA mm of a 128-dim half covers dims 8 (l%16) + mm.
//
// Every accumulator element of a lane belongs to the lane's own query, so the
// online-softmax rescale needs no data movement.  Waves merge through LDS with
// the log-sum-exp algebra of the split-KV merge; split mode writes
// (o_p, lse_p) partials.  This is the online-softmax decode over an NHD cache
// of page 1 of the source pages (issue "PagedAttnOnline is 8.1x slower per
// call", section "Where to look"), with the query heads of a KV group fused
// into one tile (page 2, PR "head_dim=128 decode arm": qg=2 fusion; here up
// to 16) and the matrix-core arm the pages leave as future work, re-designed
// for CDNA4 MFMA.
#include "pa_mfma_core.h"

namespace pa {

// ---------------------------------------------------------------------------
// Fitted partitions.  The partition size T is chosen per call from the
// sequence lengths on the device: the smallest multiple of 64 in [fit_lo,
// part_tokens] whose partitions, n_qb * sum_b ceil(L_b / T), fit in
// fit_target workgroups (part_tokens when none does).  The live (partition,
// sequence, query block) triples are then numbered partition-major, query
// block fastest -- the order of the fixed-partition grid with the dead
// triples left out -- and workgroup x takes triple x, so no workgroup of the
// grid waits behind partitions that have nothing to do.  Every wave computes
// the same result from the same lengths (lane i holds sequences i, i + 64,
// ...; at most kFitMaxBatch).  Returns false for a workgroup past the last
// triple.

// Wave-wide integer sum / maximum, every lane gets it: DPP inside 16-lane
// rows, then lane swaps across rows.
template <typename Op>
__device__ __forceinline__ int wave_reduce_i(int v, Op op) {
    v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppQuadSwap1, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppQuadSwap2, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false));
    v = op(v, __builtin_amdgcn_update_dpp(0, v, kDppRowMirror, 0xF, 0xF, false));
    auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    v = op((int)r[0], (int)r[1]);
    r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    return op((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int wave_sum_i(int v) {
    return wave_reduce_i(v, [](int a, int c) { return a + c; });
}
__device__ __forceinline__ int wave_max_i(int v) {
    return wave_reduce_i(v, [](int a, int c) { return a > c ? a : c; });
}

constexpr int kFitChunks = kFitMaxBatch / 64;

// Lane i's lengths: sequences i, i + 64, ... (0 past the batch).  Issued
// before the prologue's other reads, so they are in flight together.
__device__ __forceinline__ void fit_lengths(const DecodeParams& p, int (&len)[kFitChunks]) {
    const int lane = threadIdx.x & 63;
    const int nc = (p.B + 63) >> 6;
#pragma unroll
    for (int c = 0; c < kFitChunks; ++c) {
        const int bb = c * 64 + lane;
        len[c] = (c < nc && bb < p.B) ? p.ctx[bb] : 0;
    }
}

// The (sequence, query block, partition) triple of fitted-partition
// workgroup x and the partition size T, from the lengths of the batch: the
// smallest multiple of 64 in [fit_lo, part_tokens] that gives at most
// fit_target triples (else part_tokens), with the triples of partition j of
// all sequences ahead of those of partition j + 1.  When `hinted`, b, qb, part
// and T hold the previous call's answer on entry (decode lengths grow by one
// token per call, so it seldom changes): one round of three independent
// reductions confirms it, and only a miss runs the searches.  Returns false
// past the last triple (T is set either way).
__device__ __forceinline__ bool fit_locate(const DecodeParams& p, int x, int (&len)[kFitChunks], bool hinted, int& b,
                                           int& qb, int& part, int& T, int& L) {
    constexpr int NC = kFitChunks;
    const int lane = threadIdx.x & 63;
    const int n_qb = p.Hq / p.qw;
    const int cap = p.max_blk * p.P;
    const int nc = (p.B + 63) >> 6;
#pragma unroll
    for (int c = 0; c < NC; ++c) len[c] = clampi(len[c], 0, cap);
    // ceil(len / t) for 0 <= len < 2^24 (the host bounds the block tables
    // so), 64 <= t: len times the hardware reciprocal of t (relative error
    // near 2^-22, so under 0.1 on a quotient below 2^18) is off by at most
    // one after truncation, made exact by two integer corrections
    auto ceil_div = [](int len, int t, float rcp) {
        int d = (int)((float)len * rcp);
        d -= d * t > len ? 1 : 0;
        d += (d + 1) * t <= len ? 1 : 0;        // d = floor(len / t)
        return d + (d * t < len ? 1 : 0);
    };
    // wave-wide total times n_qb: uniform by construction; saying so keeps
    // the searches on scalar branches, so every reduction runs with the whole
    // wave active
    auto total = [&](int s) { return __builtin_amdgcn_readfirstlane(wave_sum_i(s) * n_qb); };
    auto count = [&](int t) {                   // triples with partitions of t tokens
        const float rcp = __builtin_amdgcn_rcpf((float)t);
        int s = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (c < nc) s += ceil_div(len[c], t, rcp);
        return total(s);
    };
    const int lo0 = p.fit_lo >> 6, hi0 = p.part_tokens >> 6;   // sizes in units of 64 tokens
    // n_b partitions per sequence at size T; before(j) = n_qb * sum_b min(n_b, j)
    // live triples precede partition index j
    int nb[NC];
    int n_all = -1;                             // count(T) once T is known
    int n_before = -1;                          // before(part) of the hinted part, when T is the hinted size
    if (hinted) {
        // The count only falls as the size grows, so the hinted size is the
        // answer exactly when it gives few enough triples (or is the largest
        // size) and one step below gives too many (or it is the smallest).
        const int th = T >> 6, tl = max(th - 1, 1);
        const float r_at = __builtin_amdgcn_rcpf((float)(th << 6)), r_bl = __builtin_amdgcn_rcpf((float)(tl << 6));
        int s_at = 0, s_bl = 0, s_bp = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            nb[c] = 0;
            if (c < nc) {
                nb[c] = ceil_div(len[c], th << 6, r_at);
                s_at += nb[c];
                s_bl += ceil_div(len[c], tl << 6, r_bl);
                s_bp += min(nb[c], part);
            }
        }
        const int c_at = total(s_at), c_bl = total(s_bl), bp = total(s_bp);
        if ((th == hi0 || c_at <= p.fit_target) && (th == lo0 || c_bl > p.fit_target)) {
            n_all = c_at;
            n_before = bp;
        }
    }
    if (n_all < 0) {
        int lo = lo0, hi = hi0;
        // When one step below the largest size is already too many triples,
        // the largest is the answer (the common case for batches of even
        // lengths: one probe, no search).
        if (lo < hi && count((hi - 1) << 6) > p.fit_target) lo = hi;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (count(mid << 6) <= p.fit_target) hi = mid; else lo = mid + 1;
        }
        T = __builtin_amdgcn_readfirstlane(lo << 6);
        const float rcp = __builtin_amdgcn_rcpf((float)T);
        int tot = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            nb[c] = c < nc ? ceil_div(len[c], T, rcp) : 0;
            tot += nb[c];
        }
        n_all = total(tot);
    }
    if (x >= n_all) return false;               // past the last live triple
    auto before = [&](int j) {
        int s = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (c < nc) s += min(nb[c], j);
        return total(s);
    };
    // partition index: the largest j with before(j) <= x.  The hinted part is
    // it when before(part) <= x < before(part + 1), the step between the two
    // being n_qb times the sequences with more than part partitions.
    int bx = -1;                                // before(part)
    if (n_before >= 0 && n_before <= x) {
        int more = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (c < nc) more += __builtin_popcountll(__ballot(nb[c] > part));
        if (x < n_before + n_qb * more) bx = n_before;
    }
    if (bx < 0) {
        int top = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) top = max(top, nb[c]);
        top = __builtin_amdgcn_readfirstlane(wave_max_i(top));
        int a = 0, z = top - 1;
        while (a < z) {
            const int mid = (a + z + 1) >> 1;
            if (before(mid) <= x) a = mid; else z = mid - 1;
        }
        part = a;
        bx = before(part);
    }
    const int y = x - bx;
    qb = y % n_qb;
    int k = y / n_qb;                           // the k-th sequence (from 0) with n_b > part
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c >= nc) break;
        const uint64_t m = __ballot(nb[c] > part);
        const int cnt = __builtin_popcountll(m);
        if (k < cnt) {
            const bool hit = ((m >> lane) & 1u) && __builtin_popcountll(m & ((1ull << lane) - 1ull)) == k;
            const int pos = __builtin_ctzll(__ballot(hit));
            b = c * 64 + pos;
            L = __builtin_amdgcn_readlane(len[c], pos);
            return true;
        }
        k -= cnt;
    }
    return false;
}

// ---------------------------------------------------------------------------
// Fixed partitions: one workgroup per (query block, sequence, partition of
// part_tokens tokens).  Flat grid, query block fastest and partition slowest:
// consecutive workgroups (dealt round-robin to the XCDs) cover different
// heads and sequences of the same partition index, so every XCD gets an even
// share of each sequence's work, and partitions past a sequence's end (which
// exit at once) come last.
template <int D, bool SPLIT, bool PAGE16, bool HALF, int NBUF, typename KV>
__global__ __launch_bounds__(kMBlock) void pa_decode_mfma_kernel(DecodeParams p) {
    constexpr int KK = TileFrag<D>::KK;
    constexpr int NO = D / 16;                  // O^T accumulator tiles
    const bool tracing = p.trace && (int)blockIdx.x < p.trace_wgs;   // measurement only
    uint64_t tr[4] = {tracing ? trace_clock() : 0, 0, 0, 0};
    const int qw = p.qw;                        // query heads of this workgroup (<= 16)
    const int n_qb = p.Hq / qw;
    int qb = blockIdx.x % n_qb;
    int b = (blockIdx.x / n_qb) % p.B;
    int part = blockIdx.x / n_qb / p.B;
    int T = p.part_tokens;                      // tokens per partition
    const int wave0 = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    // Fitted partitions: wave 0 reads all lengths (to locate this workgroup's
    // triple) before the hint, so both reads are in flight together.
    int len[kFitChunks];
    bool hinted = false;                        // b, qb, part, T come from a valid hint
    if (p.fit_part) {
        if (wave0 == 0) fit_lengths(p, len);
        // Fitted partitions: start from the triple this workgroup took in the
        // previous call when it is a valid one (decode lengths grow by a token
        // per step, so the plan seldom changes); else the fixed-grid slot.
        const int4 h = *reinterpret_cast<const int4*>(p.fit_hint + 4 * (int64_t)blockIdx.x);
        const int hb = __builtin_amdgcn_readfirstlane(h.x), hq = __builtin_amdgcn_readfirstlane(h.y);
        const int hp = __builtin_amdgcn_readfirstlane(h.z), ht = __builtin_amdgcn_readfirstlane(h.w);
        if (hb >= 0 && hb < p.B && hq >= 0 && hq < n_qb && ht >= p.fit_lo && ht <= p.part_tokens &&
            (ht & 63) == 0 && hp >= 0 && (int64_t)hp * ht < (int64_t)p.max_blk * p.P) {
            b = hb;
            qb = hq;
            part = hp;
            T = ht;
            hinted = true;
        }
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = wave0;                     // wave-uniform
    const int n = lane & 15, q = lane >> 4;
    auto trace_out = [&](uint32_t flags) {
        if (tracing && tid == 0) {
            uint64_t* r = p.trace + (int64_t)blockIdx.x * kTraceWords;
            r[0] = tr[0];
            r[1] = tr[1];
            r[2] = tr[2];
            r[3] = tr[3];
            r[4] = trace_clock();
            r[5] = trace_where();
            r[6] = (uint64_t)(uint32_t)b | ((uint64_t)(uint32_t)qb << 16) | ((uint64_t)(uint32_t)part << 32);
            r[7] = (uint64_t)(uint32_t)T | ((uint64_t)flags << 32);
        }
    };

    // Fitted partitions: the next call's hint (this workgroup's triple, or an
    // invalid one when it has none) and, from workgroup 0, the size chosen
    // (read by the merge kernel).  Stored once the workgroup has passed its
    // last barrier before streaming: a barrier waits for the workgroup's
    // outstanding stores, and nothing in this call reads them.
    __shared__ int s_fit[6];                    // b, qb, part, T, L, state
    auto fit_record = [&](bool none) {
        if (p.fit_part && tid == 0) {
            *reinterpret_cast<int4*>(p.fit_hint + 4 * (int64_t)blockIdx.x) =
                none ? make_int4(-1, -1, -1, -1) : make_int4(s_fit[0], s_fit[1], s_fit[2], s_fit[3]);
            if (blockIdx.x == 0) *p.fit_part = s_fit[3];
        }
    };

    // Page ids of the partition's token range are fetched without waiting for
    // the sequence length (entries past the sequence's end are never used),
    // so the two dependent reads of the prologue overlap.
    // With a window the partitions start at the window's first tile, so the
    // sequence length is needed first.
    int L = 0, t_begin = 0, t_base = 0;
    if (p.window > 0) {
        L = clampi(p.ctx[b], 0, p.max_blk * p.P);
        window_bounds(p, L, t_begin, t_base);
    }
    extern __shared__ int s_pages[];
    u32x4 qop[KK];
    int ts, pg0;
    // With fitted partitions wave 0 locates the triple while the page ids are
    // read, so the page-id loop starts at wave 1 (wave 0 takes entries only
    // past the other three waves' share).
    const int ftid = p.fit_part ? (tid + kMBlock - 64) % kMBlock : tid;
    auto fetch = [&]() {
        ts = t_base + part * T;
        int lp_hi, unused;
        page_slot(p, ts, pg0, unused);
        page_slot(p, ts + T - 1, lp_hi, unused);
        // Q does not depend on the length either: its loads go out first, so
        // they are in flight while the page ids are read and written to LDS
        // (a partition past the end drops them).
        load_q<D, HALF, KV>(p, b, qb * qw, qw, n, q, qop);
        fetch_pages(p, b, pg0, lp_hi, s_pages, ftid);
    };
    fetch();
    if (p.fit_part) {
        // Fitted partitions (never with a window).  The fetch takes the
        // hinted triple or the fixed-partition slot; when that is the triple
        // this workgroup is given, nothing is fetched again, else the fetch
        // is made again (each thread rewrites the page-id entries it wrote,
        // so no barrier is needed before the one that precedes their use).
        // Wave 0 alone reads the lengths and locates the triple (one read of
        // the lengths per workgroup) while its Q reads are in flight; the
        // others take the triple from LDS.
        if (wave == 0) {
            int fb = b, fqb = qb, fpart = part, fT = T, fL = 0;
            const bool live = fit_locate(p, (int)blockIdx.x, len, hinted, fb, fqb, fpart, fT, fL);
            if (p.fuse_ctr && blockIdx.x == 0) {
                // Merged in this kernel, a sequence with no tokens has no
                // partition and no merge to write its zero rows: this wave
                // writes them (len[] holds the clamped lengths now).
                const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < kFitChunks; ++c) {
                    uint64_t m = __ballot(c * 64 + lane < p.B && len[c] == 0);
                    while (m) {
                        const int bb = c * 64 + __builtin_ctzll(m);
                        m &= m - 1;
                        for (int idx = lane; idx < p.Hq * (D / 8); idx += 64)
                            store8(p.out, p.out_dtype, (int64_t)bb * p.o_sb + (int64_t)(idx / (D / 8)) * p.o_sh +
                                   (idx % (D / 8)) * 8, z);
                    }
                }
            }
            if (lane == 0) {
                s_fit[0] = fb;
                s_fit[1] = fqb;
                s_fit[2] = fpart;
                s_fit[3] = fT;
                s_fit[4] = fL;
                // 0: past the last triple, 1: the slot fetched, 2: another one
                s_fit[5] = !live ? 0 : (fb == b && fqb == qb && fpart == part && fT == T) ? 1 : 2;
            }
        }
        lds_barrier();
        const int state = __builtin_amdgcn_readfirstlane(s_fit[5]);
        if (state == 0) {                       // the whole workgroup
            fit_record(true);
            trace_out(1);
            return;
        }
        L = __builtin_amdgcn_readfirstlane(s_fit[4]);
        if (state == 2) {
            b = __builtin_amdgcn_readfirstlane(s_fit[0]);
            qb = __builtin_amdgcn_readfirstlane(s_fit[1]);
            part = __builtin_amdgcn_readfirstlane(s_fit[2]);
            T = __builtin_amdgcn_readfirstlane(s_fit[3]);
            fetch();
        }
    } else if (p.window <= 0) {
        L = clampi(p.ctx[b], 0, p.max_blk * p.P);
    }
    if (ts >= L && part > 0) {
        fit_record(false);
        trace_out(1);
        return;
    }
    const int h0 = qb * qw;
    const int g = h0 / (p.Hq / p.Hkv);
    const int te = min(L, ts + T);
    const bool col_live = HALF ? (n < 8 && n < qw) : (n < qw);
    // Partitions merged in this kernel (p.fuse_ctr): the group's partition
    // count (partition 0 runs even for an empty sequence); a group of one
    // partition writes its output directly, the others write partials and
    // the last of them to arrive merges them.
    const int n_used = SPLIT && p.fuse_ctr ? max(1, (L - t_base + T - 1) / T) : 0;
    const bool direct = !SPLIT || n_used == 1;
    lds_barrier();
    // Q has been in flight since the fetch (the barriers above order LDS
    // only); waiting for it here, once, keeps the wait out of the tile loop.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    if (tracing) tr[1] = trace_clock();
    fit_record(false);

    f32x4 o[NO];
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kEmptyMax, l_run = 0.f;
    LaneOffsets lo;
    lo.k = k_row<D, HALF>(0, n) * (int)p.k_ss + k_col<D, HALF>(0, n, q);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) lo.v[jj] = (4 * q + jj) * (int)p.v_ss + 8 * n;
    run_tiles<D, PAGE16, HALF, NBUF, KV>(p, s_pages, pg0, g, n, q, wave, lo, qop, col_live, ts, te, t_begin,
                                         t_begin, te, o, m_run, l_run);
    l_run = xsum32(xsum16(l_run));              // row sums over the four 16-lane rows
    if (tracing) tr[2] = trace_clock();

    __shared__ MergeLds<D> lds;
    merge_waves<D>(lds, o, m_run, l_run, qw, n, q, wave, tid,
                   [&](int jq, int d0, const float (&ov)[8], float lse) {
        const int h = h0 + jq;
        if (direct) {
            store8(p.out, p.out_dtype, (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d0, ov);
        } else {
            const int64_t slot = ((int64_t)b * p.Hq + h) * p.n_part + part;
            if (p.fuse_ctr) {
#pragma unroll
                for (int i = 0; i < 8; ++i) store_coherent(p.part_o + slot * D + d0 + i, ov[i]);
                if (d0 == 0) store_coherent(p.part_lse + slot, lse);
            } else {
                store_f32x8(p.part_o + slot * D + d0, ov);
                if (d0 == 0) p.part_lse[slot] = lse;
            }
        }
    });
    if (tracing) tr[3] = trace_clock();
    uint32_t trace_flags = 0;
    if constexpr (SPLIT) {
        if (p.fuse_ctr && n_used > 1) {
            // Count this partition in once all its partial stores are
            // complete; the partition that arrives last merges the group
            // (and sets the counter back to zero for the next call).
            __shared__ int s_last;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) {
                int* ctr = p.fuse_ctr + (b * n_qb + qb);
                const bool last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                                  n_used - 1;
                if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_last = last;
            }
            __syncthreads();
            if (__builtin_amdgcn_readfirstlane(s_last)) {
                for (int r = wave; r < qw; r += kMWaves) {
                    const int h = h0 + r;
                    merge_partials<D, true>(p, ((int64_t)b * p.Hq + h) * p.n_part, 1, n_used,
                                            (int64_t)b * p.o_sb + (int64_t)h * p.o_sh);
                }
                trace_flags = 2;
            }
        }
    }
    trace_out(trace_flags);
}

// ---------------------------------------------------------------------------
// Balanced schedule.  Order all work as the sequence of (sequence b, query
// block qb, 16-token tile) triples, sequence-major, and cut it into units
// (LeanUnits): one static unit per workgroup covering the first
// kLeanStaticNum / kLeanStaticDen of the work, then smaller dynamic units
// that workgroups take from a counter as they finish, so CUs that stream
// faster take more.  A unit may cover the end of one (b, qb) group and the
// start of others; each covered piece is one "segment".  Group G = b * n_qb
// + qb meets the units in a monotone staircase, so slot G + u names its piece
// in unit u uniquely; a piece that is a whole group is written straight to
// the output, the others as partials for the merge kernel.  Workgroups need
// the tile prefix sums of all sequences (kept in LDS); the first one also
// leaves them, with the unit sizes, in lean_meta.  Page ids are fetched
// kLeanTokensPerFill tokens at a time.
//
// The two counters (next dynamic unit, finished workgroups) start at zero;
// the last workgroup to finish sets both back to zero for the next call.

// Unit boundaries: n_wg static units of s0 tiles from 0, then dynamic units
// of s1 tiles from x_dyn = n_wg * s0 to the end (at most n_wg *
// kLeanDynPerWg of them; none when x_dyn >= total).
struct LeanUnits {
    int n_wg, s0, s1, x_dyn, n_units;
    __device__ __forceinline__ static LeanUnits plan(int total, int n_wg) {
        LeanUnits l;
        l.n_wg = n_wg;
        l.s1 = kLeanMinUnit;
        if (total < (int64_t)n_wg * kLeanDynMinPerWg) {
            // Little work per workgroup: a unit's own cost (Q and page-id
            // reads, wave merge) would outweigh the balance it buys, so the
            // static units cover everything.
            l.s0 = (total + n_wg - 1) / n_wg;
            l.x_dyn = l.s0 * n_wg;
            l.n_units = n_wg;
            return l;
        }
        l.s0 = (int)((int64_t)total * kLeanStaticNum / ((int64_t)kLeanStaticDen * n_wg));
        l.x_dyn = l.s0 * n_wg;
        const int rem = total - l.x_dyn;
        const int per = n_wg * kLeanDynPerWg;
        l.s1 = max(kLeanMinUnit, (rem + per - 1) / per);
        l.n_units = n_wg + (rem + l.s1 - 1) / l.s1;
        return l;
    }
    __device__ __forceinline__ static LeanUnits from(int s0, int s1, int n_wg) {
        LeanUnits l;
        l.n_wg = n_wg;
        l.s0 = s0;
        l.s1 = s1;
        l.x_dyn = s0 * n_wg;
        l.n_units = 0;                          // not needed to locate units
        return l;
    }
    __device__ __forceinline__ int begin(int u) const {
        return u <= n_wg ? u * s0 : x_dyn + (u - n_wg) * s1;
    }
    __device__ __forceinline__ int unit_of(int x) const {
        return x < x_dyn ? x / s0 : n_wg + (x - x_dyn) / s1;
    }
};

template <int D, bool PAGE16, bool HALF, int NBUF, typename KV>
__global__ __launch_bounds__(kMBlock) void pa_decode_mfma_lean_kernel(DecodeParams p) {
    constexpr int KK = TileFrag<D>::KK;
    constexpr int NO = D / 16;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int w = blockIdx.x;
    const int qw = p.qw;
    const int n_qb = p.Hq / qw;

    extern __shared__ int s_dyn[];
    int* s_pages = s_dyn;                       // kLeanTokensPerFill / P + 2 entries
    int* s_pref = s_dyn + p.lean_page_slots;    // B + 1 tile prefix sums

    // Tile prefix sums S[b] = sum_{b' < b} ceil((L_b' - t_base_b') / 16)
    // (t_base = 0 without a window).
    block_prefix(p.B, s_pref, [&](int bb) {
        const int L = clampi(p.ctx[bb], 0, p.max_blk * p.P);
        int t_begin, t_base;
        window_bounds(p, L, t_begin, t_base);
        return (L - t_base + kTile - 1) / kTile;
    });
    // Everything that steers the segment loop is read through readfirstlane:
    // it is wave-uniform (LDS values every lane reads alike), and saying so
    // keeps the loop on scalar branches, so the cross-lane reductions inside
    // always run with the full wave active.  Totals stay below 2^30 (the host
    // bounds the tile count).
    auto sp = [&](int i) { return __builtin_amdgcn_readfirstlane(s_pref[i]); };
    const int total = n_qb * sp(p.B);
    const LeanUnits lu = LeanUnits::plan(total, (int)gridDim.x);
    if (w == 0) {
        for (int i = tid; i <= p.B; i += kMBlock) p.lean_meta[i] = s_pref[i];
        if (tid == 0) {
            p.lean_meta[p.B + 1] = lu.s0;
            p.lean_meta[p.B + 2] = lu.s1;
            p.lean_meta[p.B + 3] = lu.n_wg;
        }
    }

    __shared__ MergeLds<D> lds;
    __shared__ int s_next[2];                    // next unit (double-buffered by iteration)
    int u = w;                                   // the static unit first
    for (int it = 0; u < lu.n_units; ++it) {
        // Thread 0 takes the next dynamic unit now and publishes it after
        // this unit's work, so the atomic's latency hides behind the work.
        int taken = 0;
        if (tid == 0) taken = atomicAdd(&p.lean_ctr[0], 1);
        int x = lu.begin(u);
        const int hi = min(total, lu.begin(u + 1));
        while (x < hi) {
            // sequence b: the last one with n_qb * S[b] <= x (empty sequences skipped)
            int lo_b = 0, hi_b = p.B - 1;
            while (lo_b < hi_b) {
                const int mid = (lo_b + hi_b + 1) >> 1;
                if (n_qb * sp(mid) <= x) lo_b = mid; else hi_b = mid - 1;
            }
            const int b = lo_b;
            const int s_b = sp(b);
            const int tiles_b = sp(b + 1) - s_b;
            const int y = x - n_qb * s_b;
            const int qb = y / tiles_b;
            const int t_lo = y - qb * tiles_b;
            const int seg_end = min(hi, n_qb * s_b + (qb + 1) * tiles_b);
            const int t_hi = t_lo + (seg_end - x);
            const bool whole = t_lo == 0 && t_hi == tiles_b;
            const int G = b * n_qb + qb;
            const int h0 = qb * qw;
            const int g = h0 / (p.Hq / p.Hkv);
            const int L = clampi(p.ctx[b], 0, p.max_blk * p.P);
            int t_begin, t_base;
            window_bounds(p, L, t_begin, t_base);
            const int ts = t_base + t_lo * kTile, te = min(t_base + t_hi * kTile, L);

            u32x4 qop[KK];
            load_q<D, HALF, KV>(p, b, h0, qw, n, q, qop);
            const bool col_live = HALF ? (n < 8 && n < qw) : (n < qw);
            f32x4 o[NO];
#pragma unroll
            for (int i = 0; i < NO; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            float m_run = kEmptyMax, l_run = 0.f;
            LaneOffsets lo;
            lo.k = k_row<D, HALF>(0, n) * (int)p.k_ss + k_col<D, HALF>(0, n, q);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) lo.v[jj] = (4 * q + jj) * (int)p.v_ss + 8 * n;
            for (int c0 = ts; c0 < te; c0 += kLeanTokensPerFill) {
                const int c1 = min(te, c0 + kLeanTokensPerFill);
                int pg0, lp1, unused;
                page_slot(p, c0, pg0, unused);
                page_slot(p, c1 - 1, lp1, unused);
                // The previous chunk's page ids must no longer be in use.  For a
                // segment's first chunk the merge (or the prologue) that ended the
                // previous one already synchronised, and skipping the barrier lets
                // the page-id reads overlap the Q reads above.
                if (c0 != ts) __syncthreads();
                fetch_pages(p, b, pg0, lp1, s_pages, tid);
                __syncthreads();
                run_tiles<D, PAGE16, HALF, NBUF, KV>(p, s_pages, pg0, g, n, q, wave, lo, qop, col_live, c0, c1,
                                                     t_begin, t_begin, c1, o, m_run, l_run);
            }
            l_run = xsum32(xsum16(l_run));
            merge_waves<D>(lds, o, m_run, l_run, qw, n, q, wave, tid,
                           [&](int jq, int d0, const float (&ov)[8], float lse) {
                const int h = h0 + jq;
                if (whole) {
                    store8(p.out, p.out_dtype, (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d0, ov);
                } else {
                    const int64_t slot = ((int64_t)(G + u)) * qw + jq;
                    store_f32x8(p.part_o + slot * D + d0, ov);
                    if (d0 == 0) p.part_lse[slot] = lse;
                }
            });
            x = seg_end;
        }
        // One barrier per unit: the slot written here is rewritten two units
        // later, after every thread has passed the next unit's barrier.
        // A counter outside [0, units left) ends the loop: only a workspace
        // whose counters did not start at zero can produce one.
        if (tid == 0) s_next[it & 1] = (taken >= 0 && taken < lu.n_units - lu.n_wg) ? lu.n_wg + taken : lu.n_units;
        __syncthreads();
        u = __builtin_amdgcn_readfirstlane(s_next[it & 1]);
    }
    // The last workgroup out resets the counters for the next call.  Every
    // workgroup has taken its last (failed) unit before it counts itself out.
    if (tid == 0 && atomicAdd(&p.lean_ctr[1], 1) == (int)gridDim.x - 1) {
        atomicExch(&p.lean_ctr[0], 0);
        atomicExch(&p.lean_ctr[1], 0);
    }
    // Sequences with no tokens still owe zero rows: the first workgroup writes them.
    if (w == 0) {
        for (int bb = 0; bb < p.B; ++bb) {
            if (s_pref[bb + 1] != s_pref[bb]) continue;
            for (int idx = tid; idx < p.Hq * (D / 8); idx += kMBlock) {
                const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                store8(p.out, p.out_dtype, (int64_t)bb * p.o_sb + (int64_t)(idx / (D / 8)) * p.o_sh +
                       (idx % (D / 8)) * 8, z);
            }
        }
    }
}

// Merge of the balanced schedule's partials: one 64-thread group per
// (head, sequence).  Groups inside a single unit were written directly.
template <int D>
__global__ __launch_bounds__(64) void pa_lean_merge_kernel(DecodeParams p) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int qw = p.qw;
    const int n_qb = p.Hq / qw;
    const int qb = h / qw, jq = h % qw;
    const int* S = p.lean_meta;
    const int tiles_b = S[b + 1] - S[b];
    if (tiles_b == 0) return;
    const LeanUnits lu = LeanUnits::from(S[p.B + 1], S[p.B + 2], S[p.B + 3]);
    const int start = n_qb * S[b] + qb * tiles_b;
    const int u0 = lu.unit_of(start), u1 = lu.unit_of(start + tiles_b - 1);
    if (u0 == u1) return;
    const int64_t G = (int64_t)b * n_qb + qb;
    merge_partials<D>(p, (G + u0) * qw + jq, qw, u1 - u0 + 1, (int64_t)b * p.o_sb + (int64_t)h * p.o_sh);
}

bool mfma_supported(int head_dim, int qw, int kv_dtype) {
    return (head_dim == 128 || head_dim == 256 || head_dim == 512) && qw >= 1 && qw <= 16 &&
           (kv_dtype == kDtBF16 || kv_dtype == kDtF16);
}

// The balanced schedule keeps the 4-wave merge buffer and the page ids of a
// whole fill in LDS: head_dim 128 and 256 only.
bool mfma_lean_supported(int head_dim, int qw, int kv_dtype) {
    return head_dim <= 256 && mfma_supported(head_dim, qw, kv_dtype);
}

template <int D, bool SPLIT, bool PAGE16, typename KV>
static hipError_t launch_mfma_t(const DecodeParams& p, int qw, hipStream_t s) {
    dim3 grid(p.fit_part ? (uint32_t)p.n_wg : (uint32_t)((int64_t)p.n_part * (p.Hq / qw) * p.B));
    // Tiles in flight per wave: three 8 KB tiles at d128, two at d256 and
    // d512 (a d512 tile is 32 KB and 128 registers; the accumulators go to
    // AGPRs, one wave per SIMD).
    constexpr int NBUF = D == 128 ? 3 : 2;
    if (qw <= 8)
        hipLaunchKernelGGL((pa_decode_mfma_kernel<D, SPLIT, PAGE16, true, NBUF, KV>), grid, dim3(kMBlock),
                           pages_lds_bytes(p), s, p);
    else
        hipLaunchKernelGGL((pa_decode_mfma_kernel<D, SPLIT, PAGE16, false, NBUF, KV>), grid, dim3(kMBlock),
                           pages_lds_bytes(p), s, p);
    return hipGetLastError();
}

// Tiles start at multiples of 16 tokens (partitions at multiples of 64); the
// one-page-per-tile path also needs in-page offsets that fit 32 bits.
static bool page16_ok(const DecodeParams& p) {
    return p.p_shift >= 4 && (int64_t)p.P * (p.k_ss > p.v_ss ? p.k_ss : p.v_ss) < (1ll << 30);
}

template <int D, typename KV>
static hipError_t launch_mfma_d(const DecodeParams& p, int qw, bool split, hipStream_t s) {
    const bool page16 = page16_ok(p);
    if (split) return page16 ? launch_mfma_t<D, true, true, KV>(p, qw, s) : launch_mfma_t<D, true, false, KV>(p, qw, s);
    return page16 ? launch_mfma_t<D, false, true, KV>(p, qw, s) : launch_mfma_t<D, false, false, KV>(p, qw, s);
}

template <int D, bool PAGE16, bool HALF, typename KV>
static hipError_t launch_lean_t(const DecodeParams& p, int n_wg, hipStream_t s) {
    constexpr int NBUF = D == 128 ? 3 : 2;
    const size_t lds = sizeof(int) * (size_t)(p.lean_page_slots + p.B + 1);
    hipLaunchKernelGGL((pa_decode_mfma_lean_kernel<D, PAGE16, HALF, NBUF, KV>), dim3(n_wg), dim3(kMBlock), lds, s,
                       p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pa_lean_merge_kernel<D>, dim3(p.Hq, p.B), dim3(64), 0, s, p);
    return hipGetLastError();
}

template <int D, typename KV>
static hipError_t launch_lean_d(const DecodeParams& p, int n_wg, hipStream_t s) {
    const bool page16 = page16_ok(p);
    const bool half = p.qw <= 8;
    if (page16)
        return half ? launch_lean_t<D, true, true, KV>(p, n_wg, s) : launch_lean_t<D, true, false, KV>(p, n_wg, s);
    return half ? launch_lean_t<D, false, true, KV>(p, n_wg, s) : launch_lean_t<D, false, false, KV>(p, n_wg, s);
}

hipError_t launch_mfma_lean(const DecodeParams& p, int head_dim, int kv_dtype, int n_wg, hipStream_t s) {
    if (!mfma_lean_supported(head_dim, p.qw, kv_dtype) || p.Hq % p.qw) return hipErrorInvalidValue;
    if (kv_dtype == kDtF16)
        return head_dim == 128 ? launch_lean_d<128, KvF16>(p, n_wg, s) : launch_lean_d<256, KvF16>(p, n_wg, s);
    return head_dim == 128 ? launch_lean_d<128, KvBF16>(p, n_wg, s) : launch_lean_d<256, KvBF16>(p, n_wg, s);
}

hipError_t launch_mfma(const DecodeParams& p, int head_dim, int kv_dtype, int qw, bool split, hipStream_t s) {
    if (!mfma_supported(head_dim, qw, kv_dtype) || p.Hq % qw) return hipErrorInvalidValue;
    if (head_dim == 512)
        return kv_dtype == kDtF16 ? launch_mfma_d<512, KvF16>(p, qw, split, s) : launch_mfma_d<512, KvBF16>(p, qw, split, s);
    if (kv_dtype == kDtF16)
        return head_dim == 128 ? launch_mfma_d<128, KvF16>(p, qw, split, s)
                               : launch_mfma_d<256, KvF16>(p, qw, split, s);
    return head_dim == 128 ? launch_mfma_d<128, KvBF16>(p, qw, split, s)
                           : launch_mfma_d<256, KvBF16>(p, qw, split, s);
}

}  // namespace pa
