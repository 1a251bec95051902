// pa_append.hip -- KV-cache append for gfx950: each sequence's newest token
// has its K and V rows (all KV heads) written into its page slot of the NHD
// pools, the step that precedes decode attention in a decode step.
//
// One workgroup per sequence; each thread moves 16-byte chunks, so a token's
// Hkv rows are written by whole-line vector stores, whatever the element
// type (bf16, fp16 or fp32: the copy is byte-exact).  The work is a few
// KB per sequence: the kernel is bound by launch and memory latency, not by
// bandwidth.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

__global__ __launch_bounds__(256) void pa_cache_append_kernel(AppendParams a) {
    const int b = blockIdx.x;
    const int L = a.ctx[b];
    if (L <= 0 || L > a.max_blk * a.P) return;      // nothing to write, or out of the table
    const int t = L - 1;
    const int lp = t / a.P, slot = t - lp * a.P;
    const int page = a.bt[(int64_t)b * a.bt_sb + lp];
    if (page < 0 || page >= a.num_pages) return;    // not a page of the pool: no write
    const int per_head = a.row_bytes / 16;          // 16-byte chunks per head row
    const int chunks = a.Hkv * per_head;            // per token (K or V)
    for (int c = threadIdx.x; c < 2 * chunks; c += blockDim.x) {
        const bool is_v = c >= chunks;
        const int cc = is_v ? c - chunks : c;
        const int g = cc / per_head, off = (cc - g * per_head) * 16;
        const char* src = is_v ? a.v_new + (int64_t)b * a.vn_sb + (int64_t)g * a.vn_sh + off
                               : a.k_new + (int64_t)b * a.kn_sb + (int64_t)g * a.kn_sh + off;
        char* dst = is_v ? a.v + (int64_t)page * a.v_sp + (int64_t)slot * a.v_ss + (int64_t)g * a.v_sh + off
                         : a.k + (int64_t)page * a.k_sp + (int64_t)slot * a.k_ss + (int64_t)g * a.k_sh + off;
        *reinterpret_cast<u32x4*>(dst) = load16(src);
    }
}

hipError_t launch_append(const AppendParams& a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(pa_cache_append_kernel, dim3(a.B), dim3(a.Hkv * a.row_bytes / 16 >= 256 ? 256 : 128), 0, s, a);
    return hipGetLastError();
}

}  // namespace pa
