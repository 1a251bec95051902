// pa_mfma_core.h -- building blocks of the gfx950 matrix-core attention
// kernels (decode and several-query): the 16-token tile loads, the MFMA tile
// step with online softmax, the register pipeline over a token range, the
// page-id fetch and the 4-wave LDS merge.  Included by the kernel sources.
#pragma once

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kMBlock = 256;
constexpr int kMWaves = kMBlock / 64;
constexpr int kTile = 16;                       // tokens per MFMA tile
constexpr float kRescaleSlack = 8.f;            // log2 units, see tile_step

template <int D>
struct TileFrag {
    static constexpr int KK = D / 32;           // Q.K MFMA steps
    static constexpr int VH = D / 128;          // 128-dim halves of a V row
    u32x4 k[KK];
    u32x4 v[4][VH];
};

// Element offset of token t's row (KV head g) in a pool with strides sp, ss, sh.
__device__ __forceinline__ int64_t row_offset(const DecodeParams& p, const int* s_pages, int pg0,
                                              int t, int64_t sp, int64_t ss, int64_t gsh) {
    int lp, slot;
    page_slot(p, t, lp, slot);
    return (int64_t)s_pages[lp - pg0] * sp + (int64_t)slot * ss + gsh;
}

// Per-lane 32-bit element offsets inside one page, fixed for the whole
// kernel: the lane's K row and chunk, and the four V rows 4q + jj (chunk n).
struct LaneOffsets {
    int k;
    int v[4];
};

// K row (token offset inside the tile) and element offset inside the row of
// load i (0 .. D/32 - 1) of lane (n, q).
template <int D, bool HALF>
__device__ __forceinline__ int k_row(int i, int n) {
    if constexpr (HALF) return (i / (D / 64)) * 8 + (n & 7);
    else return n;
}
template <int D, bool HALF>
__device__ __forceinline__ int k_col(int i, int n, int q) {
    if constexpr (HALF) return 64 * (i % (D / 64)) + 32 * (n >> 3) + 8 * q;
    else return 32 * i + 8 * q;
}

// Issue the loads of the 16-token tile starting at tb.  K: see k_row/k_col
// (A operand layout); V: tokens tb + 4q + jj, 16 lanes per row.  Tokens
// outside [t_min, te) -- past the end, or before a window -- are clamped to
// the nearest row inside it and masked out of the softmax, so nothing
// outside is read (a weight of 0 times a non-finite row would not vanish).
// PAGE16: the page size is a power of two >= 16, so the tile lies in one
// page; the page base is wave-uniform and each lane adds a fixed 32-bit
// offset.
template <int D, bool PAGE16, bool HALF>
__device__ __forceinline__ void load_tile(const DecodeParams& p, const int* s_pages, int pg0, int g,
                                          int n, int q, const LaneOffsets& lo, int tb, int t_min,
                                          int te, TileFrag<D>& f) {
    constexpr int KK = TileFrag<D>::KK;
    if constexpr (PAGE16) {
        const int lp = tb >> p.p_shift;
        const int page = __builtin_amdgcn_readfirstlane(s_pages[lp - pg0]);
        const int slot0 = tb - (lp << p.p_shift);
        const uint16_t* kt = static_cast<const uint16_t*>(p.k) + (int64_t)page * p.k_sp + (int64_t)g * p.k_sh +
                             (int64_t)slot0 * p.k_ss;
        const uint16_t* vt = static_cast<const uint16_t*>(p.v) + (int64_t)page * p.v_sp + (int64_t)g * p.v_sh +
                             (int64_t)slot0 * p.v_ss;
        const int ks = (int)p.k_ss, vs = (int)p.v_ss;
        if (tb + kTile <= te && tb >= t_min) {  // full tile (wave-uniform)
#pragma unroll
            for (int i = 0; i < KK; ++i) {
                const int extra = HALF ? (i / (D / 64)) * 8 * ks + 64 * (i % (D / 64)) : 32 * i;
                f.k[i] = load16_nt(kt + lo.k + extra);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int hh = 0; hh < TileFrag<D>::VH; ++hh)
                    f.v[jj][hh] = load16_nt(vt + lo.v[jj] + 128 * hh);
        } else {                                // edge tile: clamp rows into [t_min, te)
            const int first = max(t_min - tb, 0), last = te - 1 - tb;
#pragma unroll
            for (int i = 0; i < KK; ++i)
                f.k[i] = load16_nt(kt + clampi(k_row<D, HALF>(i, n), first, last) * ks + k_col<D, HALF>(i, n, q));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int vo = clampi(4 * q + jj, first, last) * vs + 8 * n;
#pragma unroll
                for (int hh = 0; hh < TileFrag<D>::VH; ++hh) f.v[jj][hh] = load16_nt(vt + vo + 128 * hh);
            }
        }
    } else {
        const int64_t gk = (int64_t)g * p.k_sh, gv = (int64_t)g * p.v_sh;
#pragma unroll
        for (int i = 0; i < KK; ++i) {
            const int tk = clampi(tb + k_row<D, HALF>(i, n), t_min, te - 1);
            f.k[i] = load16_nt(static_cast<const uint16_t*>(p.k) + row_offset(p, s_pages, pg0, tk, p.k_sp, p.k_ss, gk) +
                               k_col<D, HALF>(i, n, q));
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int tv = clampi(tb + 4 * q + jj, t_min, te - 1);
            const uint16_t* vr = static_cast<const uint16_t*>(p.v) + row_offset(p, s_pages, pg0, tv, p.v_sp, p.v_ss, gv) +
                                 8 * n;
#pragma unroll
            for (int hh = 0; hh < TileFrag<D>::VH; ++hh) f.v[jj][hh] = load16_nt(vr + 128 * hh);
        }
    }
}

__device__ __forceinline__ float xmax16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Value of lane l + 32 (meaningful in lanes 0..31) / of lane l - 32 (in 32..63).
__device__ __forceinline__ float from_hi32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[1]);
}
__device__ __forceinline__ float from_lo32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]);
}
constexpr int kDppRowRor8 = 0x128;    // row_ror:8 (lane i <- lane (i + 8) mod 16)

__device__ __forceinline__ float xsum16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 16-token tile: logits on MFMA, online-softmax update, O^T += V^T P^T.
template <int D, bool HALF, typename KV>
__device__ __forceinline__ void tile_step(const DecodeParams& p, const TileFrag<D>& cur,
                                          const u32x4 (&qop)[D / 32], int tb, int mask_lo, int mask_hi,
                                          int q, bool col_live, f32x4 (&o)[D / 16], float& m_run,
                                          float& l_run) {
    constexpr int KK = TileFrag<D>::KK;
    constexpr int VH = TileFrag<D>::VH;
    constexpr int NO = D / 16;
    // logits: lane (n, q) ends with query n, tokens tb + 4q + r; the tokens
    // of column n outside [mask_lo, mask_hi) (per lane) are masked out
    f32x4 s;
    if constexpr (HALF) {
        constexpr int KH = D / 64;
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) {
            c0 = KV::mma_qk(cur.k[kk], qop[kk], c0);
            c1 = KV::mma_qk(cur.k[KH + kk], qop[kk], c1);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // (token, half 0) sits in lane (n, q<2), (token, half 1) in lane (n+8, q+2)
            // Every cross-lane move runs with all 64 lanes active: evaluate
            // both candidates first, then select (a conditional operand would
            // become a branch, and a lane swap under a partial exec mask reads
            // inactive lanes).
            const float f0 = c0[r] + dpp_mov<kDppRowRor8>(from_hi32(c0[r]));
            const float f1 = c1[r] + dpp_mov<kDppRowRor8>(from_hi32(c1[r]));
            const float f1_lo = from_lo32(f1);
            s[r] = q < 2 ? f0 : f1_lo;
        }
    } else {
        s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            s = KV::mma_qk(cur.k[kk], qop[kk], s);
    }
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = tb + 4 * q + r;
        sv[r] = (col_live && t < mask_hi && t >= mask_lo) ? s[r] * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, sv[r]);
    }
    mt = xmax32(xmax16(mt));
    // The reference max only moves when the tile max exceeds it by more than
    // kRescaleSlack (log2 units): p = 2^(s - m) then stays <= 2^kRescaleSlack,
    // exact in fp32 and bf16 alike, and the accumulator rescale (a
    // wave-uniform branch) runs only a handful of times per partition.
    if (__any(mt > m_run + kRescaleSlack)) {
        const float mn = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - mn);
        m_run = mn;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NO; ++i) o[i] *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sv[r] - m_run);
    // P.V takes P in the KV type, as the sum of two such values: hi = P
    // rounded, lo = (P - hi) rounded.  The weights are then exact to about
    // 2^-17 relative (2^-22 for fp16) instead of the 2^-9 of one rounding,
    // so the output is close to correctly rounded.  The path is bound by
    // the K/V reads; the second P.V MFMA per dim block costs no time there.
    // The normaliser sums the same hi + lo.
    const u32x2 ph = {KV::pack2(pr[0], pr[1]), KV::pack2(pr[2], pr[3])};
    const u32x2 pl = {KV::pack2(pr[0] - KV::lo(ph[0]), pr[1] - KV::hi(ph[0])),
                      KV::pack2(pr[2] - KV::lo(ph[1]), pr[3] - KV::hi(ph[1]))};
    l_run += ((KV::lo(ph[0]) + KV::hi(ph[0])) + (KV::lo(ph[1]) + KV::hi(ph[1]))) +
             ((KV::lo(pl[0]) + KV::hi(pl[0])) + (KV::lo(pl[1]) + KV::hi(pl[1])));

    // O^T += V^T . P^T, V transposed in registers (4 tokens x 8 dims per lane)
#pragma unroll
    for (int hh = 0; hh < VH; ++hh)
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) {
            // (token 0, token 1) and (token 2, token 3) of dim 8n + mm: the low
            // (even mm) or high (odd mm) halves of dword mm/2 of two rows.
            const int x = mm >> 1;
            const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
            const u32x2 va = {__builtin_amdgcn_perm(cur.v[1][hh][x], cur.v[0][hh][x], sel),
                              __builtin_amdgcn_perm(cur.v[3][hh][x], cur.v[2][hh][x], sel)};
            o[hh * 8 + mm] = KV::mma_pv(va, pl, KV::mma_pv(va, ph, o[hh * 8 + mm]));
        }
}

// Q^T as the B operand of query heads h0 .. h0 + qw - 1 of sequence b (same
// k <-> dim map as the K rows of the layout), in the KV element type: a Q
// stored in another type is converted (round to nearest even).  Lanes of
// columns past qw load head h0 instead and are not cleared: an output column
// depends only on its own column of Q^T and those columns' logits are masked
// out, and a clear would make the wave wait for the reads right here.  In the
// split layout the operands past the loaded ones are zero.
template <int D, bool HALF, typename KV>
__device__ __forceinline__ void load_q(const DecodeParams& p, int b, int h0, int qw, int n, int q,
                                       u32x4 (&qop)[D / 32]) {
    const int qcol = HALF ? (n & 7) : n;
    const bool live = qcol < qw;
    const int64_t qr = (int64_t)b * p.q_sb + (int64_t)(h0 + (live ? qcol : 0)) * p.q_sh;
    constexpr int NL = HALF ? D / 64 : D / 32;          // loads; the split layout leaves the rest unused
    u32x4 w[NL];
    // The type test stays outside the loops, so all the loads are in flight
    // together (a test per load would make each wait for the one before).
    if (p.q_dtype == KV::code) {
#pragma unroll
        for (int kk = 0; kk < NL; ++kk) w[kk] = load16(static_cast<const uint16_t*>(p.q) + qr + k_col<D, HALF>(kk, n, q));
    } else {
#pragma unroll
        for (int kk = 0; kk < NL; ++kk) {
            float f[8];
            load8f(p.q, p.q_dtype, qr + k_col<D, HALF>(kk, n, q), f);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[kk][i] = KV::pack2(f[2 * i], f[2 * i + 1]);
        }
    }
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        qop[kk] = kk < NL ? w[kk < NL ? kk : 0] : u32x4{0u, 0u, 0u, 0u};
}

// This wave's share of the tokens [ts, te): tiles ts + 16 (wave + 4k), rows
// loaded from [t_min, te), softmax masked per lane to [mask_lo, mask_hi).  The
// page ids of the range sit in s_pages from logical page pg0 on.  NBUF
// register buffers rotate so NBUF - 1 tiles' loads are in flight while one
// is consumed; the steady-state loop issues its prefetches unconditionally
// (each wait covers exactly the tile being consumed) and the last few tiles
// drain in a short unrolled tail.  No data moves between buffers.
template <int D, bool PAGE16, bool HALF, int NBUF, typename KV>
__device__ __forceinline__ void run_tiles(const DecodeParams& p, const int* s_pages, int pg0, int g,
                                          int n, int q, int wave, const LaneOffsets& lo,
                                          const u32x4 (&qop)[D / 32], bool col_live, int ts, int te,
                                          int t_min, int mask_lo, int mask_hi, f32x4 (&o)[D / 16],
                                          float& m_run, float& l_run) {
    const int n_tiles = (max(te - ts, 0) + kTile - 1) / kTile;
    const int n_my = n_tiles > wave ? (n_tiles - wave + kMWaves - 1) / kMWaves : 0;
    auto tile_tb = [&](int k) { return ts + (wave + k * kMWaves) * kTile; };
    TileFrag<D> fb[NBUF];
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
        if (i < n_my) load_tile<D, PAGE16, HALF>(p, s_pages, pg0, g, n, q, lo, tile_tb(i), t_min, te, fb[i]);
    int k = 0;
    for (; k + 2 * NBUF - 2 < n_my; k += NBUF) {
#pragma unroll
        for (int i = 0; i < NBUF; ++i) {
            load_tile<D, PAGE16, HALF>(p, s_pages, pg0, g, n, q, lo, tile_tb(k + i + NBUF - 1), t_min, te,
                                       fb[(i + NBUF - 1) % NBUF]);
            __builtin_amdgcn_sched_barrier(0);
            tile_step<D, HALF, KV>(p, fb[i], qop, tile_tb(k + i), mask_lo, mask_hi, q, col_live, o, m_run, l_run);
        }
    }
#pragma unroll
    for (int i = 0; i < 2 * NBUF - 1; ++i) {
        if (k + i < n_my) {
            if (k + i + NBUF - 1 < n_my)
                load_tile<D, PAGE16, HALF>(p, s_pages, pg0, g, n, q, lo, tile_tb(k + i + NBUF - 1), t_min, te,
                                           fb[(i + NBUF - 1) % NBUF]);
            tile_step<D, HALF, KV>(p, fb[i % NBUF], qop, tile_tb(k + i), mask_lo, mask_hi, q, col_live, o, m_run,
                                      l_run);
        }
    }
}

// Page ids of logical pages [lp0, lp1] of sequence b into s_pages (whole
// workgroup; the caller synchronises before use).
template <int NT = kMBlock>
__device__ __forceinline__ void fetch_pages(const DecodeParams& p, int b, int lp0, int lp1, int* s_pages,
                                            int tid) {
    lp1 = min(lp1, p.max_blk - 1);
    const int32_t* btrow = p.bt + (int64_t)b * p.bt_sb;
    for (int i = tid; i <= lp1 - lp0; i += NT) s_pages[i] = clampi(btrow[lp0 + i], 0, p.num_pages - 1);
}

template <int D>
struct MergeLds {
    float o[kMWaves][16][D + 4];                // +4: spread the 16 query rows over banks
    float m[kMWaves][16], l[kMWaves][16];
};

// Merge the 4 waves' online-softmax states through LDS and hand each
// (query jq, 8 dims at d0) chunk, normalised, with its log-sum-exp, to emit().
// O^T tile (hh, mm), element r of lane (n, q) holds query n, dim
// 128 hh + 32 q + 8 r + mm.  Ends with the workgroup synchronised.
template <int D, typename Emit>
__device__ __forceinline__ void merge_waves(MergeLds<D>& lds, const f32x4 (&o)[D / 16], float m_run,
                                            float l_run, int qw, int n, int q, int wave, int tid,
                                            Emit emit) {
    constexpr int VH = D / 128;
    if (n < qw) {
#pragma unroll
        for (int hh = 0; hh < VH; ++hh)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int mm = 0; mm < 8; ++mm)
                    lds.o[wave][n][128 * hh + 32 * q + 8 * r + mm] = o[hh * 8 + mm][r];
        if (q == 0) {
            lds.m[wave][n] = m_run;
            lds.l[wave][n] = l_run;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < qw * (D / 8); idx += kMBlock) {
        const int jq = idx / (D / 8);
        const int d0 = (idx % (D / 8)) * 8;
        float M = lds.m[0][jq];
#pragma unroll
        for (int w = 1; w < kMWaves; ++w) M = fmaxf(M, lds.m[w][jq]);
        float wt[kMWaves], lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kMWaves; ++w) {
            wt[w] = fast_exp2(lds.m[w][jq] - M);
            lsum += lds.l[w][jq] * wt[w];
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        float ov[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float a = 0.f;
#pragma unroll
            for (int w = 0; w < kMWaves; ++w) a = fmaf(lds.o[w][jq][d0 + i], wt[w], a);
            ov[i] = a * inv;
        }
        emit(jq, d0, ov, lsum > 0.f ? M + __log2f(lsum) : -INFINITY);
    }
    __syncthreads();
}

__device__ __forceinline__ void store_f32x8(float* dst, const float (&v)[8]) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Exclusive prefix sums s_pref[b] = sum_{b' < b} value(b') for b in [0, n]
// into LDS, by the whole workgroup of NT threads (every thread calls it), NT
// entries per pass: a shuffle scan inside each wave, then across the waves.
template <int NT = kMBlock, typename F>
__device__ __forceinline__ void block_prefix(int n, int* s_pref, F value) {
    __shared__ int s_carry;
    __shared__ int s_wsum[NT / 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid == 0) {
        s_carry = 0;
        s_pref[0] = 0;
    }
    __syncthreads();
    for (int c = 0; c < n; c += NT) {
        const int bb = c + tid;
        int v = bb < n ? value(bb) : 0;
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(v, off);
            if (lane >= off) v += t;
        }
        if (lane == 63) s_wsum[wave] = v;
        __syncthreads();
        int before = s_carry;
        for (int i = 0; i < wave; ++i) before += s_wsum[i];
        if (bb < n) s_pref[bb + 1] = before + v;
        __syncthreads();
        if (tid == 0) s_carry = s_pref[min(c + NT, n)];
        __syncthreads();
    }
}

}  // namespace pa
