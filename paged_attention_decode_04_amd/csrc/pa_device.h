// pa_device.h -- device-side helpers and the launch parameter block shared by
// the gfx950 decode kernels.  Wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything a decode kernel needs, passed by value (kernarg segment).
// Strides are in elements.
struct DecodeParams {
    const uint16_t* q;      int64_t q_sb, q_sh;             // [B][Hq][D]
    const uint16_t* k;      int64_t k_sp, k_ss, k_sh;       // [NP][P][Hkv][D]
    const uint16_t* v;      int64_t v_sp, v_ss, v_sh;
    const int32_t*  bt;     int64_t bt_sb;                  // [B][MaxBlk]
    const int32_t*  ctx;                                    // [B]
    uint16_t*       out;    int64_t o_sb, o_sh;             // [B][Hq][D]
    float*          part_o;                                 // [B][Hq][n_part][D]
    float*          part_lse;                               // [B][Hq][n_part]
    int   B, Hq, Hkv, P, max_blk, num_pages;
    int   p_shift;                                          // log2(P) if P is a power of 2, else -1
    int   part_tokens;                                      // tokens per partition
    int   n_part;                                           // grid partitions
    int   qw;                                               // query heads per workgroup
    int*  lean_meta;                                        // balanced schedule: S[0..B], s0, s1, n_wg
    int*  lean_ctr;                                         // balanced schedule: next unit, finished WGs
    int   lean_page_slots;                                  // balanced schedule: page-id LDS entries
    int   window;                                           // 0 = none, else the last `window` tokens
    float scale_log2;                                       // scale * log2(e)
};

// KV-cache append: newest token of each sequence into its page slot.
struct AppendParams {
    const uint16_t* k_new; const uint16_t* v_new;           // [B, Hkv, D]
    int64_t kn_sb, kn_sh, vn_sb, vn_sh;                     // their batch and head strides
    uint16_t* k; uint16_t* v;                               // pools [NP, P, Hkv, D]
    int64_t k_sp, k_ss, k_sh, v_sp, v_ss, v_sh;
    const int32_t* bt; int64_t bt_sb;
    const int32_t* ctx;
    int B, Hkv, D, P, max_blk, num_pages;
};

constexpr float kLog2e = 1.4426950408889634f;
// Finite "no token yet" running maximum: exp2(kEmptyMax - kEmptyMax) == 1 and
// exp2(-inf - kEmptyMax) == 0, so empty states merge without NaNs.
constexpr float kEmptyMax = -1.0e30f;

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Data-parallel-primitive lane moves inside a 16-lane row (gfx9 DPP controls).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror (i <-> 7-i in each 8)
constexpr int kDppRowMirror = 0x140;  // row_mirror      (i <-> 15-i in each 16)

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<kDppQuadSwap1>(x);
    x += dpp_mov<kDppQuadSwap2>(x);
    x += dpp_mov<kDppHalfMirror>(x);
    x += dpp_mov<kDppRowMirror>(x);
    return x;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Streaming load: K/V rows are read once per call, keep them out of the way.
__device__ __forceinline__ u32x4 load16_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Logical page index and slot of token t (P a power of two takes shifts).
// First attended token t_begin (the window keeps [L - window, L)) and the
// start t_base of the work, t_begin rounded down to a 16-token tile: kernels
// walk [t_base, L) in tiles and mask the tokens below t_begin.
__device__ __forceinline__ void window_bounds(const DecodeParams& p, int L, int& t_begin, int& t_base) {
    t_begin = (p.window > 0 && L > p.window) ? L - p.window : 0;
    t_base = t_begin & ~15;
}

__device__ __forceinline__ void page_slot(const DecodeParams& p, int t, int& lp, int& slot) {
    if (p.p_shift >= 0) {
        lp = t >> p.p_shift;
        slot = t & ((1 << p.p_shift) - 1);
    } else {
        lp = t / p.P;
        slot = t - lp * p.P;
    }
}

// Log-sum-exp merge of n split partials (o_p fp32 rows of D, lse_p base 2)
// at slots first, first + step, ... into one bf16 output row, by 64 threads
// holding D / 64 elements each.  Partials are read four at a time with
// their lse and o rows together, so a merge of up to four costs one round
// trip to memory; the running maximum rescales between batches.  n == 0
// writes zeros.
template <int D>
__device__ __forceinline__ void merge_partials(const DecodeParams& p, int64_t first, int64_t step, int n,
                                               uint16_t* orow) {
    constexpr int EPT = D / 64;
    typedef float vec_t __attribute__((ext_vector_type(EPT)));
    const int t = threadIdx.x;
    float M = -INFINITY, wsum = 0.f;
    vec_t o = {};
    for (int i0 = 0; i0 < n; i0 += 4) {
        float l[4];
        vec_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = min(i0 + j, n - 1);           // in range; extra entries are ignored
            const int64_t slot = first + (int64_t)i * step;
            l[j] = i0 + j < n ? p.part_lse[slot] : -INFINITY;
            v[j] = *reinterpret_cast<const vec_t*>(p.part_o + slot * D + t * EPT);
        }
        const float mb = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
        if (mb == -INFINITY) continue;
        const float mn = fmaxf(M, mb);
        const float a = fast_exp2(M - mn);
        wsum *= a;
        o *= a;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float w = fast_exp2(l[j] - mn);
            wsum += w;
            o += w * v[j];
        }
        M = mn;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int e = 0; e < EPT; e += 2)
        *reinterpret_cast<uint32_t*>(orow + t * EPT + e) = pack_bf16x2(o[e] * inv, o[e + 1] * inv);
}

}  // namespace pa
