// pa_device.h -- device-side helpers and the launch parameter block shared by
// the gfx950 decode kernels.  Wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Element types (the ABI's PA_DTYPE_* codes).
constexpr int kDtBF16 = 1, kDtF32 = 3, kDtF16 = 4;

// Everything a decode kernel needs, passed by value (kernarg segment).
// Strides are in elements of each tensor's own type.
struct DecodeParams {
    const void*     q;      int64_t q_sb, q_sh;             // [B][Hq][D], type q_dtype
    const void*     k;      int64_t k_sp, k_ss, k_sh;       // [NP][P][Hkv][D], the kernel's KV type
    const void*     v;      int64_t v_sp, v_ss, v_sh;
    const int32_t*  bt;     int64_t bt_sb;                  // [B][MaxBlk]
    const int32_t*  ctx;                                    // [B]
    void*           out;    int64_t o_sb, o_sh;             // [B][Hq][D], type out_dtype
    int             q_dtype, out_dtype;
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
    const int32_t* qstart;                                  // several queries: rows of sequence b [B + 1]
    int   q_rows;                                           // several queries: rows of q and out
    int   n_slots;                                          // several queries: query-block slots in the grid
    int*  fit_part;                                         // fitted partitions: the size chosen on the device
                                                            // (written by workgroup 0, read by the merge); else null
    int   fit_lo;                                           // fitted partitions: smallest size (multiple of 64)
    int   fit_target;                                       // fitted partitions: workgroups live partitions may fill
    int   n_wg;                                             // fitted partitions: workgroups in the grid
    int*  fit_hint;                                         // fitted partitions: [n_wg][4] triple (b, query
                                                            // block, partition, size) each workgroup took in
                                                            // the previous call (a hint: checked before use)
    int*  fuse_ctr;                                         // partitions merged in the decode kernel: one
                                                            // arrival counter per (sequence, query block),
                                                            // zero between calls; null = separate merge kernel
    float scale_log2;                                       // scale * log2(e)
    uint64_t* trace;                                        // measurement: kTraceWords stamps per workgroup
                                                            // of the partitioned MFMA decode, or null
    int   trace_wgs;                                        // workgroups the trace buffer holds
};

// Workgroup barrier that orders LDS only.  The plain barrier's release fence
// waits for every vector memory operation in flight (loads included); this one
// waits for the wave's LDS operations alone, so global loads issued before it
// (Q rows, the next tile) stay in flight across it.  For exchanges through LDS
// only: global memory written before it is not made visible to the workgroup.
// s_waitcnt operand that waits for every vector memory operation of the wave
// (vmcnt 0) and for nothing else (expcnt 7, lgkmcnt 15: their maxima).
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-workgroup timeline record of the partitioned matrix-core decode (a
// measurement aid): [0] entry, [1] prologue done (lengths, page ids, Q), [2]
// wave 0's streaming done, [3] wave merge and stores done, [4] exit, in
// s_memrealtime ticks (the device's wall-clock rate); [5] HW_ID | XCC_ID << 32; [6] sequence |
// query block << 16 | partition << 32; [7] partition tokens | flags << 32
// (flag 1: no partition to run, 2: merged its group in the kernel).
constexpr int kTraceWords = 8;
__device__ __forceinline__ uint64_t trace_clock() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint64_t trace_where() {
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);     // HW_REG_HW_ID, 32 bits
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // HW_REG_XCC_ID, 32 bits
    return (uint64_t)hw | ((uint64_t)xcc << 32);
}

// KV-cache append: newest token of each sequence into its page slot.  Byte
// pointers and byte strides: the copy does not depend on the element type.
struct AppendParams {
    const char* k_new; const char* v_new;                   // [B, Hkv, D]
    int64_t kn_sb, kn_sh, vn_sb, vn_sh;                     // their batch and head strides (bytes)
    char* k; char* v;                                       // pools [NP, P, Hkv, D]
    int64_t k_sp, k_ss, k_sh, v_sp, v_ss, v_sh;             // bytes
    const int32_t* bt; int64_t bt_sb;
    const int32_t* ctx;
    int B, Hkv, row_bytes, P, max_blk, num_pages;           // row_bytes = D * element size
};

constexpr float kLog2e = 1.4426950408889634f;
// Finite "no token yet" running maximum: exp2(kEmptyMax - kEmptyMax) == 1 and
// exp2(-inf - kEmptyMax) == 0, so empty states merge without NaNs.
constexpr float kEmptyMax = -1.0e30f;

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats to a bf16 pair (lo in the low half) with one v_cvt_pk_bf16_f32:
// round to nearest, ties to even, denormals kept; a NaN stays a NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// IEEE binary16 halves of a dword, and fp32 -> binary16 (round to nearest even).
__device__ __forceinline__ float f16lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
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

template <typename T>
__device__ __forceinline__ u32x4 load16(const T* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Streaming load: K/V rows are read once per call, keep them out of the way.
template <typename T>
__device__ __forceinline__ u32x4 load16_nt(const T* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 8 consecutive elements of an array of element type dt, as floats (the
// element offset is a multiple of 8, so every load is 16-byte aligned).
__device__ __forceinline__ void load8f(const void* base, int dt, int64_t off, float (&f)[8]) {
    if (dt == kDtF32) {
        const float* fp = static_cast<const float*>(base) + off;
        const u32x4 a = load16(fp), b = load16(fp + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = __uint_as_float(a[i]);
            f[4 + i] = __uint_as_float(b[i]);
        }
        return;
    }
    const u32x4 w = load16(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = dt == kDtF16 ? f16lo(w[i]) : bf16lo(w[i]);
        f[2 * i + 1] = dt == kDtF16 ? f16hi(w[i]) : bf16hi(w[i]);
    }
}

// 8 floats stored at element offset off of an array of type dt (rounded to
// nearest even for the 16-bit types); off is a multiple of 8.
__device__ __forceinline__ void store8(void* base, int dt, int64_t off, const float (&v)[8]) {
    if (dt == kDtF32) {
        float* fp = static_cast<float*>(base) + off;
        *reinterpret_cast<float4*>(fp) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(fp + 4) = make_float4(v[4], v[5], v[6], v[7]);
        return;
    }
    u32x4 pk;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        pk[i] = dt == kDtF16 ? pack_f16x2(v[2 * i], v[2 * i + 1]) : pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + off) = pk;
}

// 2 floats at element offset off (even) of an array of type dt.
__device__ __forceinline__ void store2(void* base, int dt, int64_t off, float a, float b) {
    if (dt == kDtF32) {
        *reinterpret_cast<float2*>(static_cast<float*>(base) + off) = make_float2(a, b);
        return;
    }
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + off) =
        dt == kDtF16 ? pack_f16x2(a, b) : pack_bf16x2(a, b);
}

// 16-bit KV element types on the matrix cores: the Q.K and P.V MFMAs and
// the packing of P (and of a converted Q) into that type.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct KvBF16 {
    static constexpr int code = kDtBF16;
    __device__ static __forceinline__ f32x4 mma_qk(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mma_pv(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                        __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
    __device__ static __forceinline__ float lo(uint32_t u) { return bf16lo(u); }
    __device__ static __forceinline__ float hi(uint32_t u) { return bf16hi(u); }
};

struct KvF16 {
    static constexpr int code = kDtF16;
    __device__ static __forceinline__ f32x4 mma_qk(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mma_pv(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                    __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return pack_f16x2(lo, hi); }
    __device__ static __forceinline__ float lo(uint32_t u) { return f16lo(u); }
    __device__ static __forceinline__ float hi(uint32_t u) { return f16hi(u); }
};

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

// Partials that another workgroup merges in the same kernel (on any XCD, so
// through any L2): stored and loaded as relaxed agent-scope atomics, i.e.
// written through to and read from the device's point of coherence.
// Ordering comes from waiting for the stores (s_waitcnt 0) before the
// arrival count is taken, and from the count being read before the loads.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Running log-sum-exp merge of split partials (o_p fp32 rows of D, lse_p
// base 2), by 64 threads (lane = threadIdx.x % 64) holding D / 64 elements
// each.  Partials are added four at a time, with their lse and o rows read
// together; the running maximum rescales between batches.  COHERENT: the
// partials were written in the same kernel (load_coherent).
template <int D, bool COHERENT = false>
struct LseMerge {
    static constexpr int EPT = D / 64;
    typedef float vec_t __attribute__((ext_vector_type(EPT)));
    float M = -INFINITY, wsum = 0.f;
    vec_t o = {};

    // Read slots first + (i0 + j) * step, j < 4, clamped to slot n_read - 1
    // (n_read >= 1 slots exist there).
    __device__ __forceinline__ static void read(const DecodeParams& p, int64_t first, int64_t step, int i0,
                                                int n_read, float (&l)[4], vec_t (&v)[4]) {
        const int t = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t slot = first + (int64_t)min(i0 + j, n_read - 1) * step;
            if constexpr (COHERENT) {
                l[j] = load_coherent(p.part_lse + slot);
#pragma unroll
                for (int e = 0; e < EPT; ++e) v[j][e] = load_coherent(p.part_o + slot * D + t * EPT + e);
            } else {
                l[j] = p.part_lse[slot];
                v[j] = *reinterpret_cast<const vec_t*>(p.part_o + slot * D + t * EPT);
            }
        }
    }
    // Add the first `live` (0..4) of a batch; the others are ignored whatever
    // they hold (selected away, never multiplied by a zero weight).
    __device__ __forceinline__ void add(const float (&l)[4], const vec_t (&v)[4], int live) {
        float lj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) lj[j] = j < live ? l[j] : -INFINITY;
        const float mb = fmaxf(fmaxf(lj[0], lj[1]), fmaxf(lj[2], lj[3]));
        if (mb == -INFINITY) return;
        const float mn = fmaxf(M, mb);
        const float a = fast_exp2(M - mn);
        wsum *= a;
        o *= a;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float w = fast_exp2(lj[j] - mn);      // 0 for an ignored slot
            wsum += w;
            const vec_t add = w * v[j];
            o = j < live ? o + add : o;
        }
        M = mn;
    }
    // Batches from partial i0 on, up to partial n.
    __device__ __forceinline__ void add_range(const DecodeParams& p, int64_t first, int64_t step, int i0, int n) {
        for (; i0 < n; i0 += 4) {
            float l[4];
            vec_t v[4];
            read(p, first, step, i0, n, l, v);
            add(l, v, n - i0);
        }
    }
    // Normalised row into the output at element offset out_off (n == 0 writes zeros).
    __device__ __forceinline__ void store(const DecodeParams& p, int64_t out_off) const {
        const int t = threadIdx.x & 63;
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
        for (int e = 0; e < EPT; e += 2)
            store2(p.out, p.out_dtype, out_off + t * EPT + e, o[e] * inv, o[e + 1] * inv);
    }
};

// Log-sum-exp merge of n split partials at slots first, first + step, ...
// into the output row at element offset out_off (in the output's type).  The
// first 16 partials (8 at head_dim 512) are all read before any is added:
// one round trip to memory for them.
template <int D, bool COHERENT = false>
__device__ __forceinline__ void merge_partials(const DecodeParams& p, int64_t first, int64_t step, int n,
                                               int64_t out_off) {
    constexpr int NB = D <= 256 ? 4 : 2;        // batches of four read at once
    typedef LseMerge<D, COHERENT> M;
    M m;
    float l[NB][4];
    typename M::vec_t v[NB][4];
    if (n > 0) {
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (4 * k < n) M::read(p, first, step, 4 * k, n, l[k], v[k]);
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (4 * k < n) m.add(l[k], v[k], n - 4 * k);
    }
    m.add_range(p, first, step, 4 * NB, n);
    m.store(p, out_off);
}

}  // namespace pa
