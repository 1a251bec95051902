// pa_probe.hip -- streaming-read probes (include/pa_probe.h): the bytes of a
// decode call, read with no arithmetic, as the bandwidth reference of the
// decode kernels.  Reads only; the one store is conditional on a value the
// folded loads practically never take.
#include <hip/hip_runtime.h>

#include "pa_mfma_core.h"
#include "pa_probe.h"

namespace {

constexpr uint32_t kSinkMagic = 0x9e3779b9u;
constexpr int kProbeBlock = 256;
constexpr int kProbeFill = 4096;                // tokens whose page ids one LDS fill holds

__device__ __forceinline__ uint32_t fold(const pa::u32x4& v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

template <int U>
__global__ __launch_bounds__(kProbeBlock) void pa_probe_contig_kernel(const char* base, int64_t n16,
                                                                      uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeBlock;
    int64_t i = (int64_t)blockIdx.x * kProbeBlock + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        pa::u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = pa::load16_nt(base + (i + u * stride) * 16);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
    }
    for (; i < n16; i += stride) acc ^= fold(pa::load16_nt(base + i * 16));
    if (acc == kSinkMagic) sink[blockIdx.x] = acc;
}

struct PagedProbe {
    const char* k;
    const char* v;
    int64_t k_sp, k_ss, k_sh, v_sp, v_ss, v_sh;   // bytes
    const int32_t* bt;
    int64_t bt_sb;
    const int32_t* ctx;
    int B, Hkv, P, p_shift, num_pages, max_blk, page_slots;
    uint32_t* sink;
};

// One 16-token tile of K and V rows (ROW16 16-byte chunks each) of KV head g
// over tokens [tb, tb + 16), rows past te - 1 clamped to te - 1 (so nothing
// outside the sequence is read).  Chunk j * 64 + lane of the tile's 16 x
// ROW16 chunks goes to the lane: whole rows per 16 or 32 lanes.
template <int ROW16>
struct ProbeTile {
    static constexpr int N = 16 * ROW16 / 64;
    pa::u32x4 k[N], v[N];
};

template <int ROW16>
__device__ __forceinline__ void probe_load(const PagedProbe& pp, const int* s_pages, int pg0, int g, int lane,
                                           int tb, int te, ProbeTile<ROW16>& f) {
#pragma unroll
    for (int j = 0; j < ProbeTile<ROW16>::N; ++j) {
        const int idx = j * 64 + lane;
        const int t = min(tb + idx / ROW16, te - 1);
        const int c = idx % ROW16;
        const int lp = t >> pp.p_shift;
        const int slot = t & (pp.P - 1);
        const int64_t page = s_pages[lp - pg0];
        f.k[j] = pa::load16_nt(pp.k + page * pp.k_sp + (int64_t)slot * pp.k_ss + (int64_t)g * pp.k_sh + c * 16);
        f.v[j] = pa::load16_nt(pp.v + page * pp.v_sp + (int64_t)slot * pp.v_ss + (int64_t)g * pp.v_sh + c * 16);
    }
}

template <int ROW16>
__device__ __forceinline__ uint32_t probe_fold(const ProbeTile<ROW16>& f) {
    uint32_t a = 0;
#pragma unroll
    for (int j = 0; j < ProbeTile<ROW16>::N; ++j) a ^= fold(f.k[j]) ^ fold(f.v[j]);
    return a;
}

template <int ROW16, int NBUF>
__global__ __launch_bounds__(kProbeBlock) void pa_probe_paged_kernel(PagedProbe pp) {
    extern __shared__ int s_dyn[];
    int* s_pages = s_dyn;                       // pp.page_slots entries
    int* s_pref = s_dyn + pp.page_slots;        // B + 1 tile prefix sums
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cap = pp.max_blk * pp.P;
    pa::block_prefix(pp.B, s_pref, [&](int bb) { return (pa::clampi(pp.ctx[bb], 0, cap) + 15) / 16; });
    auto sp = [&](int i) { return __builtin_amdgcn_readfirstlane(s_pref[i]); };
    const int total = pp.Hkv * sp(pp.B);
    const int per = (total + (int)gridDim.x - 1) / (int)gridDim.x;
    int x = (int)blockIdx.x * per;
    const int hi = min(total, x + per);
    uint32_t acc = 0;
    while (x < hi) {
        int lo_b = 0, hi_b = pp.B - 1;          // the last b with Hkv * S[b] <= x
        while (lo_b < hi_b) {
            const int mid = (lo_b + hi_b + 1) >> 1;
            if (pp.Hkv * sp(mid) <= x) lo_b = mid; else hi_b = mid - 1;
        }
        const int b = lo_b;
        const int tiles_b = sp(b + 1) - sp(b);
        const int y = x - pp.Hkv * sp(b);
        const int g = y / tiles_b;
        const int t_lo = y - g * tiles_b;
        const int seg_end = min(hi, pp.Hkv * sp(b) + (g + 1) * tiles_b);
        const int L = pa::clampi(pp.ctx[b], 0, cap);
        const int ts = t_lo * 16, te = min((t_lo + seg_end - x) * 16, L);
        for (int c0 = ts; c0 < te; c0 += kProbeFill) {
            const int c1 = min(te, c0 + kProbeFill);
            const int pg0 = c0 >> pp.p_shift, lp1 = (c1 - 1) >> pp.p_shift;
            __syncthreads();                    // the previous fill is no longer read
            const int32_t* row = pp.bt + (int64_t)b * pp.bt_sb;
            for (int i = tid; i <= lp1 - pg0; i += kProbeBlock) s_pages[i] = pa::clampi(row[pg0 + i], 0, pp.num_pages - 1);
            __syncthreads();
            const int n_tiles = (c1 - c0 + 15) / 16;
            const int n_my = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;
            auto tb = [&](int k) { return c0 + (wave + 4 * k) * 16; };
            ProbeTile<ROW16> fb[NBUF];
#pragma unroll
            for (int i = 0; i < NBUF - 1; ++i)
                if (i < n_my) probe_load<ROW16>(pp, s_pages, pg0, g, lane, tb(i), c1, fb[i]);
            int k = 0;
            for (; k + 2 * NBUF - 2 < n_my; k += NBUF) {
#pragma unroll
                for (int i = 0; i < NBUF; ++i) {
                    probe_load<ROW16>(pp, s_pages, pg0, g, lane, tb(k + i + NBUF - 1), c1, fb[(i + NBUF - 1) % NBUF]);
                    acc ^= probe_fold<ROW16>(fb[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 2 * NBUF - 1; ++i) {
                if (k + i < n_my) {
                    if (k + i + NBUF - 1 < n_my)
                        probe_load<ROW16>(pp, s_pages, pg0, g, lane, tb(k + i + NBUF - 1), c1, fb[(i + NBUF - 1) % NBUF]);
                    acc ^= probe_fold<ROW16>(fb[i % NBUF]);
                }
            }
        }
        x = seg_end;
    }
    if (acc == kSinkMagic) pp.sink[blockIdx.x] = acc;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Issue-rate probe: every round, NM matrix-core products (16x16x32 bf16, on
// two accumulator chains) and NV independent fp32 FMAs (on eight chains).
// MIXED: every wave issues both, interleaved in program order.  Otherwise
// the waves of a workgroup alternate between MFMA only and FMA only (each
// SIMD then holds waves of both kinds).  Nothing is read from memory; the
// folded result goes to the sink only if it equals a fixed constant.
typedef float pf32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));

template <int NM, int NV, bool MIXED>
__global__ __launch_bounds__(kProbeBlock) void pa_probe_issue_kernel(uint32_t* sink, float seed, int rounds) {
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    pbf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
        b[i] = (__bf16)(seed - (float)i);
    }
    pf32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = seed * (float)i + (float)threadIdx.x;
    auto mfmas = [&]() {
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[m & 1], 0, 0, 0);
    };
    auto fmas = [&]() {
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j & 7] = fmaf(v[j & 7], 1.0001f, 0.5f);
    };
    if constexpr (MIXED) {
        for (int it = 0; it < rounds; ++it) {
            mfmas();
            fmas();
        }
    } else if ((wave + (int)blockIdx.x) & 1) {      // wave-uniform
        for (int it = 0; it < rounds; ++it) mfmas();
    } else {
        for (int it = 0; it < rounds; ++it) fmas();
    }
    float s = acc[0][0] + acc[1][1];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
    if (__float_as_uint(s) == kSinkMagic) sink[blockIdx.x] = kSinkMagic;
}

struct IssueMode {
    int nm, nv, mixed;
};
// The menu of pa_probe_issue: one MFMA or four FMAs alone, one MFMA with 2,
// 3, 4 and 8 FMAs, two MFMAs with 6, all in every wave; then MFMA-only
// beside FMA-only waves.
constexpr IssueMode kIssueModes[] = {{1, 0, 1}, {0, 4, 1}, {1, 2, 1}, {1, 3, 1}, {1, 4, 1},
                                     {1, 8, 1}, {2, 6, 1}, {1, 4, 0}, {2, 6, 0}};
constexpr int kIssueModeCount = sizeof(kIssueModes) / sizeof(kIssueModes[0]);

template <int NM, int NV, bool MIXED>
void launch_issue(int n_wg, int rounds, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL((pa_probe_issue_kernel<NM, NV, MIXED>), dim3(n_wg), dim3(kProbeBlock), 0, s, sink, 1.0f,
                       rounds);
}

}  // namespace

extern "C" {

int pa_probe_read_contiguous(const void* base, int64_t bytes, int n_wg, void* sink, void* stream) {
    if (!base || !sink || !aligned16(base) || bytes < 0 || bytes % 16 || n_wg < 1 || n_wg > 65536) return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(pa_probe_contig_kernel<4>, dim3(n_wg), dim3(kProbeBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<const char*>(base), bytes / 16, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int pa_probe_read_paged(const pa_probe_paged* d, int n_wg, void* sink, void* stream) {
    if (!d || !sink || !d->k || !d->v || !d->block_tables || !d->context_lens) return 1;
    if (d->row_bytes != 256 && d->row_bytes != 512) return 1;
    if (d->batch < 1 || d->batch > 4096 || d->num_kv_heads < 1 || d->num_pages < 1 || d->max_blocks < 1) return 1;
    if (d->page_size < 16 || (d->page_size & (d->page_size - 1))) return 1;
    if ((int64_t)d->max_blocks * d->page_size > (1 << 30) || d->bt_sb < d->max_blocks) return 1;
    const int64_t st[6] = {d->k_sp, d->k_ss, d->k_sh, d->v_sp, d->v_ss, d->v_sh};
    for (int64_t s : st)
        if (s < 0 || s % 16) return 1;
    if (!aligned16(d->k) || !aligned16(d->v) || n_wg < 1 || n_wg > 4096) return 1;
    // (Hkv x tiles) must stay below 2^31: at most 2^30 / 16 tiles per sequence
    if ((int64_t)d->num_kv_heads * d->batch * ((int64_t)d->max_blocks * d->page_size / 16) >= ((int64_t)1 << 31))
        return 1;
    PagedProbe pp{};
    pp.k = static_cast<const char*>(d->k);
    pp.v = static_cast<const char*>(d->v);
    pp.k_sp = d->k_sp; pp.k_ss = d->k_ss; pp.k_sh = d->k_sh;
    pp.v_sp = d->v_sp; pp.v_ss = d->v_ss; pp.v_sh = d->v_sh;
    pp.bt = d->block_tables;
    pp.bt_sb = d->bt_sb;
    pp.ctx = d->context_lens;
    pp.B = d->batch;
    pp.Hkv = d->num_kv_heads;
    pp.P = d->page_size;
    pp.p_shift = __builtin_ctz((unsigned)d->page_size);
    pp.num_pages = d->num_pages;
    pp.max_blk = d->max_blocks;
    pp.page_slots = kProbeFill / d->page_size + 2;
    pp.sink = static_cast<uint32_t*>(sink);
    const size_t lds = sizeof(int) * (size_t)(pp.page_slots + pp.B + 1);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (d->row_bytes == 256)
        hipLaunchKernelGGL((pa_probe_paged_kernel<16, 3>), dim3(n_wg), dim3(kProbeBlock), lds, s, pp);
    else
        hipLaunchKernelGGL((pa_probe_paged_kernel<32, 2>), dim3(n_wg), dim3(kProbeBlock), lds, s, pp);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int pa_probe_issue_modes(int mode, int* nm, int* nv, int* mixed) {
    if (mode < 0) return kIssueModeCount;
    if (mode >= kIssueModeCount || !nm || !nv || !mixed) return -1;
    *nm = kIssueModes[mode].nm;
    *nv = kIssueModes[mode].nv;
    *mixed = kIssueModes[mode].mixed;
    return kIssueModeCount;
}

int pa_probe_issue(int mode, int n_wg, int rounds, void* sink, void* stream) {
    if (!sink || mode < 0 || mode >= kIssueModeCount || n_wg < 1 || n_wg > 65536 || rounds < 1 ||
        rounds > (1 << 20))
        return 1;
    uint32_t* sk = static_cast<uint32_t*>(sink);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (mode) {
        case 0: launch_issue<1, 0, true>(n_wg, rounds, sk, s); break;
        case 1: launch_issue<0, 4, true>(n_wg, rounds, sk, s); break;
        case 2: launch_issue<1, 2, true>(n_wg, rounds, sk, s); break;
        case 3: launch_issue<1, 3, true>(n_wg, rounds, sk, s); break;
        case 4: launch_issue<1, 4, true>(n_wg, rounds, sk, s); break;
        case 5: launch_issue<1, 8, true>(n_wg, rounds, sk, s); break;
        case 6: launch_issue<2, 6, true>(n_wg, rounds, sk, s); break;
        case 7: launch_issue<1, 4, false>(n_wg, rounds, sk, s); break;
        default: launch_issue<2, 6, false>(n_wg, rounds, sk, s); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
