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

// K/V element types on the vector ALUs: a 16-byte load holds PER elements;
// lane c of a 16-lane row holds dims 8c .. 8c + 7 of every 128-dim block.
struct VkBF16 {
    using E = uint16_t;
    static constexpr int PER = 8;
    __device__ static __forceinline__ void to_f(u32x4 w, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16lo(w[i]);
            f[2 * i + 1] = bf16hi(w[i]);
        }
    }
};
struct VkF16 {
    using E = uint16_t;
    static constexpr int PER = 8;
    __device__ static __forceinline__ void to_f(u32x4 w, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = f16lo(w[i]);
            f[2 * i + 1] = f16hi(w[i]);
        }
    }
};
struct VkF32 {
    using E = float;
    static constexpr int PER = 4;
    __device__ static __forceinline__ void to_f(u32x4 w, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
    }
};

template <int D, int U, typename KV>
struct RowFrag {
    static constexpr int NCH = D / 128;         // 128-dim blocks per row
    static constexpr int LPC = 8 / KV::PER;     // 16-byte loads per block per lane
    u32x4 k[U][NCH * LPC];
    u32x4 v[U][NCH * LPC];
    bool valid[U];
};

template <int D, int U, typename KV>
__device__ __forceinline__ void load_rows(const DecodeParams& p, const int* s_pages, int pg0,
                                          int g, int c, int t_first, int te, int ts, int t_min,
                                          RowFrag<D, U, KV>& f) {
    using E = typename KV::E;
    constexpr int LPC = RowFrag<D, U, KV>::LPC;
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
        const E* kp = static_cast<const E*>(p.k) + page * p.k_sp + (int64_t)slot * p.k_ss + (int64_t)g * p.k_sh + c * 8;
        const E* vp = static_cast<const E*>(p.v) + page * p.v_sp + (int64_t)slot * p.v_ss + (int64_t)g * p.v_sh + c * 8;
#pragma unroll
        for (int ch = 0; ch < RowFrag<D, U, KV>::NCH; ++ch)
#pragma unroll
            for (int j = 0; j < LPC; ++j) {
                f.k[u][ch * LPC + j] = load16_nt(kp + ch * 128 + j * KV::PER);
                f.v[u][ch * LPC + j] = load16_nt(vp + ch * 128 + j * KV::PER);
            }
    }
}

template <int D, int QW, int U, bool SPLIT, typename KV>
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

    // Q rows of the group (any element type), pre-scaled to base-2 logits.
    float qf[QW][E];
#pragma unroll
    for (int j = 0; j < QW; ++j) {
        const int64_t qrow = (int64_t)b * p.q_sb + (int64_t)(h0 + j) * p.q_sh + c * 8;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            float f[8];
            load8f(p.q, p.q_dtype, qrow + ch * 128, f);
#pragma unroll
            for (int i = 0; i < 8; ++i) qf[j][ch * 8 + i] = f[i] * p.scale_log2;
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
    RowFrag<D, U, KV> cur;
    if (n_tok > 0) load_rows<D, U, KV>(p, s_pages, pg0, g, c, ts + my_row, te, ts, t_begin, cur);
    for (int base = 0; base < n_tok; base += TPI) {
        RowFrag<D, U, KV> nxt;
        const bool more = base + TPI < n_tok;
        if (more) load_rows<D, U, KV>(p, s_pages, pg0, g, c, ts + base + TPI + my_row, te, ts, t_begin, nxt);

        float s[U][QW];
        float vf[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[E];
            constexpr int LPC = RowFrag<D, U, KV>::LPC;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                for (int j = 0; j < LPC; ++j) {
                    KV::to_f(cur.k[u][ch * LPC + j], &kf[ch * 8 + j * KV::PER]);
                    KV::to_f(cur.v[u][ch * LPC + j], &vf[u][ch * 8 + j * KV::PER]);
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
            store8(p.out, p.out_dtype, (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d0, o);
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
// Partials read before the row's count is known: 32 at head_dim 128 (5
// registers each), 8 above, where a slot is 1-2 KB: slots past the row's
// count are read for nothing, and at 16 those bytes cost more than the
// second round trip that rows of more than 8 partitions take.
template <int D>
constexpr int kMergeEager = D == 128 ? 32 : 8;
template <int D>
__global__ __launch_bounds__(64) void pa_lse_merge_kernel(DecodeParams p) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t first = ((int64_t)b * p.Hq + h) * p.n_part;
    // The partials of up to kMergeEager<D> slots (those of the n_part slots that
    // exist) are all read with the length, not after it: one round trip to
    // memory per row.  Slots past the row's count are read and ignored.
    constexpr int NB = kMergeEager<D> / 4;
    LseMerge<D> m;
    float l[NB][4];
    typename LseMerge<D>::vec_t v[NB][4];
#pragma unroll
    for (int k = 0; k < NB; ++k)
        if (4 * k < p.n_part) LseMerge<D>::read(p, first, 1, 4 * k, p.n_part, l[k], v[k]);
    // fitted partitions: the size the decode kernel chose for this call
    const int T = p.fit_part ? *p.fit_part : p.part_tokens;
    const int L = clampi(p.ctx[b], 0, p.max_blk * p.P);
    int t_begin, t_base;
    window_bounds(p, L, t_begin, t_base);
    const int n_used = min((L - t_base + T - 1) / T, p.n_part);
#pragma unroll
    for (int k = 0; k < NB; ++k)
        if (4 * k < n_used) m.add(l[k], v[k], n_used - 4 * k);
    m.add_range(p, first, 1, kMergeEager<D>, n_used);
    m.store(p, (int64_t)b * p.o_sb + (int64_t)h * p.o_sh);
}

// ------------------------------------------------------------------ launch
template <int D, int QW, int U, bool SPLIT, typename KV>
static hipError_t launch_valu_t(const DecodeParams& p, size_t lds, hipStream_t s) {
    dim3 grid(p.n_part, p.Hq / QW, p.B);
    hipLaunchKernelGGL((pa_decode_valu_kernel<D, QW, U, SPLIT, KV>), grid, dim3(kBlock), lds, s, p);
    return hipGetLastError();
}

template <int D, int QW, int U, typename KV>
static hipError_t launch_valu_s(const DecodeParams& p, bool split, size_t lds, hipStream_t s) {
    return split ? launch_valu_t<D, QW, U, true, KV>(p, lds, s) : launch_valu_t<D, QW, U, false, KV>(p, lds, s);
}

template <int D, typename KV>
static hipError_t launch_valu_d(const DecodeParams& p, int qw, bool split, size_t lds, hipStream_t s) {
    if constexpr (D == 512) {
        // 32 dims per lane per query: at most two queries per workgroup fit
        // the registers.
        switch (qw) {
            case 1: return launch_valu_s<D, 1, 1, KV>(p, split, lds, s);
            case 2: return launch_valu_s<D, 2, 1, KV>(p, split, lds, s);
            default: return hipErrorInvalidValue;
        }
    } else {
        constexpr int U = D == 128 ? 2 : 1;
        switch (qw) {
            case 1: return launch_valu_s<D, 1, 2, KV>(p, split, lds, s);
            case 2: return launch_valu_s<D, 2, 2, KV>(p, split, lds, s);
            case 4: return launch_valu_s<D, 4, U, KV>(p, split, lds, s);
            case 8: return launch_valu_s<D, 8, U, KV>(p, split, lds, s);
            default: return hipErrorInvalidValue;
        }
    }
}

template <typename KV>
static hipError_t launch_valu_k(const DecodeParams& p, int head_dim, int qw, bool split, hipStream_t s) {
    const size_t lds = pages_lds_bytes(p);
    if (head_dim == 128) return launch_valu_d<128, KV>(p, qw, split, lds, s);
    if (head_dim == 256) return launch_valu_d<256, KV>(p, qw, split, lds, s);
    if (head_dim == 512) return launch_valu_d<512, KV>(p, qw, split, lds, s);
    return hipErrorInvalidValue;
}

bool valu_supported(int head_dim, int qw, int kv_dtype) {
    const bool kv_ok = kv_dtype == kDtBF16 || kv_dtype == kDtF16 || kv_dtype == kDtF32;
    if (head_dim == 512) return kv_ok && (qw == 1 || qw == 2);
    return kv_ok && (head_dim == 128 || head_dim == 256) && (qw == 1 || qw == 2 || qw == 4 || qw == 8);
}

hipError_t launch_valu(const DecodeParams& p, int head_dim, int kv_dtype, int qw, bool split, hipStream_t s) {
    if (!valu_supported(head_dim, qw, kv_dtype)) return hipErrorInvalidValue;
    if (kv_dtype == kDtF16) return launch_valu_k<VkF16>(p, head_dim, qw, split, s);
    if (kv_dtype == kDtF32) return launch_valu_k<VkF32>(p, head_dim, qw, split, s);
    return launch_valu_k<VkBF16>(p, head_dim, qw, split, s);
}

hipError_t launch_merge(const DecodeParams& p, int head_dim, hipStream_t s) {
    dim3 grid(p.Hq, p.B);
    if (head_dim == 128)
        hipLaunchKernelGGL(pa_lse_merge_kernel<128>, grid, dim3(64), 0, s, p);
    else if (head_dim == 256)
        hipLaunchKernelGGL(pa_lse_merge_kernel<256>, grid, dim3(64), 0, s, p);
    else if (head_dim == 512)
        hipLaunchKernelGGL(pa_lse_merge_kernel<512>, grid, dim3(64), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
