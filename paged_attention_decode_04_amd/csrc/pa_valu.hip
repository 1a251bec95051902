// pa_valu.hip -- vector-ALU decode paged-attention kernel for gfx950 (wave64).
//
// One workgroup (256 threads = 4 waves) handles one sequence b, one block of
// QW query heads that share KV head g, and one partition of the sequence's
// tokens.  Each K/V row (D bf16 = 256 or 512 bytes) is read by a 16-lane DPP
// row with one 128-bit load per lane per 128 dims, so a wave streams 4 whole
// rows per load instruction and every byte of a row is used.  The QW queries
// of the group are evaluated against each loaded row (grouped-query fusion:
// one read of a KV row serves all its query heads).
//
// Softmax runs online in fp32 on base-2 logits (Q is pre-scaled by
// scale*log2 e): each 16-lane row keeps its own running max m, sum l and
// accumulator over the tokens it sees; rows are merged inside the wave with
// lane shuffles and across waves through LDS, using the same log-sum-exp
// algebra as the split-KV merge kernel.  This is the online-softmax decode of
// page 1 of the source pages (issue "PagedAttnOnline is 8.1x slower per
// call", section "Where to look") with the warp-split reduction order of
// page 3 (PR "head_dim-128 arm for the warp-split-KV decode kernel"),
// re-laid out for 64-wide waves.
//
// Split mode writes per-partition (o_p = acc / l, lse_p = m + log2 l) for the
// merge kernel instead of bf16 output.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kRowsPerWave = 4;                 // 16 lanes per row
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;

template <int D, int U>
struct RowFrag {
    static constexpr int NCH = D / 128;         // 16-byte chunks per lane per row
    u32x4 k[U][NCH];
    u32x4 v[U][NCH];
    bool valid[U];
};

template <int D, int U>
__device__ __forceinline__ void load_rows(const DecodeParams& p, const int* s_pages, int pg0,
                                          int g, int c, int t_first, int te, int ts, int t_min,
                                          RowFrag<D, U>& f) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int t = t_first + u * kRowsPerBlock;
        f.valid[u] = t < te && t >= t_min;
        // Masked rows read a token inside [t_min, te) instead: a weight of 0
        // times a row outside (past L, or before the window) need not vanish.
        const int tt = f.valid[u] ? t : max(ts, t_min);
        int lp, slot;
        page_slot(p, tt, lp, slot);
        const int64_t page = s_pages[lp - pg0];
        const uint16_t* kp = p.k + page * p.k_sp + (int64_t)slot * p.k_ss + (int64_t)g * p.k_sh + c * 8;
        const uint16_t* vp = p.v + page * p.v_sp + (int64_t)slot * p.v_ss + (int64_t)g * p.v_sh + c * 8;
#pragma unroll
        for (int ch = 0; ch < RowFrag<D, U>::NCH; ++ch) {
            f.k[u][ch] = load16_nt(kp + ch * 128);
            f.v[u][ch] = load16_nt(vp + ch * 128);
        }
    }
}

template <int D, int QW, int U, bool SPLIT>
__global__ __launch_bounds__(kBlock) void pa_decode_valu_kernel(DecodeParams p) {
    constexpr int E = D / 16;                   // dims held per lane
    constexpr int NCH = E / 8;
    const int part = blockIdx.x;
    const int h0 = blockIdx.y * QW;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int row = lane >> 4, c = lane & 15;
    const int qg = p.Hq / p.Hkv;
    const int g = h0 / qg;

    const int L = clampi(p.ctx[b], 0, p.max_blk * p.P);
    int t_begin, t_base;
    window_bounds(p, L, t_begin, t_base);
    const int ts = t_base + part * p.part_tokens;
    if (ts >= L && part > 0) return;            // unused partition (merge skips it)
    const int te = min(L, ts + p.part_tokens);
    const int n_tok = max(te - ts, 0);

    // Page ids of this partition, fetched once (the block-table walk).
    extern __shared__ int s_pages[];
    int pg0 = 0;
    if (n_tok > 0) {
        int lp_last, slot_unused;
        page_slot(p, ts, pg0, slot_unused);
        page_slot(p, te - 1, lp_last, slot_unused);
        const int32_t* btrow = p.bt + (int64_t)b * p.bt_sb;
        for (int i = tid; i <= lp_last - pg0; i += kBlock)
            s_pages[i] = clampi(btrow[pg0 + i], 0, p.num_pages - 1);
    }

    // Q rows of the group, pre-scaled to base-2 logits.
    float qf[QW][E];
#pragma unroll
    for (int j = 0; j < QW; ++j) {
        const uint16_t* qrow = p.q + (int64_t)b * p.q_sb + (int64_t)(h0 + j) * p.q_sh + c * 8;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            const u32x4 w = load16(qrow + ch * 128);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qf[j][ch * 8 + 2 * i] = bf16lo(w[i]) * p.scale_log2;
                qf[j][ch * 8 + 2 * i + 1] = bf16hi(w[i]) * p.scale_log2;
            }
        }
    }
    __syncthreads();

    float m[QW], l[QW], acc[QW][E];
#pragma unroll
    for (int j = 0; j < QW; ++j) {
        m[j] = kEmptyMax;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[j][e] = 0.f;
    }

    constexpr int TPI = kRowsPerBlock * U;      // tokens per iteration per workgroup
    const int my_row = wave * kRowsPerWave + row;
    RowFrag<D, U> cur;
    if (n_tok > 0) load_rows<D, U>(p, s_pages, pg0, g, c, ts + my_row, te, ts, t_begin, cur);
    for (int base = 0; base < n_tok; base += TPI) {
        RowFrag<D, U> nxt;
        const bool more = base + TPI < n_tok;
        if (more) load_rows<D, U>(p, s_pages, pg0, g, c, ts + base + TPI + my_row, te, ts, t_begin, nxt);

        float s[U][QW];
        float vf[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[E];
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kf[ch * 8 + 2 * i] = bf16lo(cur.k[u][ch][i]);
                    kf[ch * 8 + 2 * i + 1] = bf16hi(cur.k[u][ch][i]);
                    vf[u][ch * 8 + 2 * i] = bf16lo(cur.v[u][ch][i]);
                    vf[u][ch * 8 + 2 * i + 1] = bf16hi(cur.v[u][ch][i]);
                }
#pragma unroll
            for (int j = 0; j < QW; ++j) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) d = fmaf(qf[j][e], kf[e], d);
                d = row16_sum(d);
                s[u][j] = cur.valid[u] ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < QW; ++j) {
            float mx = s[0][j];
#pragma unroll
            for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][j]);
            const float mn = fmaxf(m[j], mx);
            const float alpha = fast_exp2(m[j] - mn);
            m[j] = mn;
            l[j] *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[j][e] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float pr = fast_exp2(s[u][j] - mn);
                l[j] += pr;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[j][e] = fmaf(pr, vf[u][e], acc[j][e]);
            }
        }
        if (more) cur = nxt;
    }

    // Merge the 4 rows of each wave (lanes 16 and 32 apart hold the same dims).
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
        for (int j = 0; j < QW; ++j) {
            const float mo = __shfl_xor(m[j], off);
            const float lo = __shfl_xor(l[j], off);
            const float mn = fmaxf(m[j], mo);
            const float a = fast_exp2(m[j] - mn), bw = fast_exp2(mo - mn);
            l[j] = l[j] * a + lo * bw;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[j][e] = acc[j][e] * a + __shfl_xor(acc[j][e], off) * bw;
            m[j] = mn;
        }
    }

    // Merge the waves through LDS.
    __shared__ float s_acc[kWaves][QW][D];
    __shared__ float s_m[kWaves][QW], s_l[kWaves][QW];
    if (row == 0) {
#pragma unroll
        for (int j = 0; j < QW; ++j) {
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                for (int i = 0; i < 8; ++i) s_acc[wave][j][ch * 128 + c * 8 + i] = acc[j][ch * 8 + i];
            if (c == 0) {
                s_m[wave][j] = m[j];
                s_l[wave][j] = l[j];
            }
        }
    }
    __syncthreads();

    for (int idx = tid; idx < QW * (D / 8); idx += kBlock) {
        const int j = idx / (D / 8);
        const int d0 = (idx % (D / 8)) * 8;
        float M = s_m[0][j];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][j]);
        float wt[kWaves], lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            wt[w] = fast_exp2(s_m[w][j] - M);
            lsum += s_l[w][j] * wt[w];
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float a = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) a = fmaf(s_acc[w][j][d0 + i], wt[w], a);
            o[i] = a * inv;
        }
        const int h = h0 + j;
        if constexpr (!SPLIT) {
            u32x4 pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
            *reinterpret_cast<u32x4*>(p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d0) = pk;
        } else {
            const int64_t slot = ((int64_t)b * p.Hq + h) * p.n_part + part;
            float* op = p.part_o + slot * D + d0;
            *reinterpret_cast<float4*>(op) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(op + 4) = make_float4(o[4], o[5], o[6], o[7]);
            if (d0 == 0) p.part_lse[slot] = lsum > 0.f ? M + __log2f(lsum) : -INFINITY;
        }
    }
}

// Log-sum-exp merge of the split-KV partials: one 64-thread group per (h, b).
template <int D>
__global__ __launch_bounds__(64) void pa_lse_merge_kernel(DecodeParams p) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int L = clampi(p.ctx[b], 0, p.max_blk * p.P);
    int t_begin, t_base;
    window_bounds(p, L, t_begin, t_base);
    const int n_used = (L - t_base + p.part_tokens - 1) / p.part_tokens;
    merge_partials<D>(p, ((int64_t)b * p.Hq + h) * p.n_part, 1, n_used,
                      p.out + (int64_t)b * p.o_sb + (int64_t)h * p.o_sh);
}

// ------------------------------------------------------------------ launch
template <int D, int QW, int U, bool SPLIT>
static hipError_t launch_valu_t(const DecodeParams& p, size_t lds, hipStream_t s) {
    dim3 grid(p.n_part, p.Hq / QW, p.B);
    hipLaunchKernelGGL((pa_decode_valu_kernel<D, QW, U, SPLIT>), grid, dim3(kBlock), lds, s, p);
    return hipGetLastError();
}

template <int D, int QW, int U>
static hipError_t launch_valu_s(const DecodeParams& p, bool split, size_t lds, hipStream_t s) {
    return split ? launch_valu_t<D, QW, U, true>(p, lds, s) : launch_valu_t<D, QW, U, false>(p, lds, s);
}

template <int D>
static hipError_t launch_valu_d(const DecodeParams& p, int qw, bool split, size_t lds, hipStream_t s) {
    constexpr int U = D == 128 ? 2 : 1;
    switch (qw) {
        case 1: return launch_valu_s<D, 1, 2>(p, split, lds, s);
        case 2: return launch_valu_s<D, 2, 2>(p, split, lds, s);
        case 4: return launch_valu_s<D, 4, U>(p, split, lds, s);
        case 8: return launch_valu_s<D, 8, U>(p, split, lds, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_valu(const DecodeParams& p, int head_dim, int qw, bool split, hipStream_t s) {
    const size_t lds = pages_lds_bytes(p);
    if (head_dim == 128) return launch_valu_d<128>(p, qw, split, lds, s);
    if (head_dim == 256) return launch_valu_d<256>(p, qw, split, lds, s);
    return hipErrorInvalidValue;
}

hipError_t launch_merge(const DecodeParams& p, int head_dim, hipStream_t s) {
    dim3 grid(p.Hq, p.B);
    if (head_dim == 128)
        hipLaunchKernelGGL(pa_lse_merge_kernel<128>, grid, dim3(64), 0, s, p);
    else if (head_dim == 256)
        hipLaunchKernelGGL(pa_lse_merge_kernel<256>, grid, dim3(64), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
