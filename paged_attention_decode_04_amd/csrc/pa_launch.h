// pa_launch.h -- host-side launch entry points of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_device.h"

namespace pa {

// Dynamic LDS holding one partition's page ids: a partition of T tokens spans
// at most ceil(T / P) + 1 pages.
inline size_t pages_lds_bytes(const DecodeParams& p) {
    return sizeof(int) * (size_t)((p.part_tokens + p.P - 1) / p.P + 1);
}

// Vector-ALU decode kernel; qw = query heads per workgroup (1, 2, 4 or 8;
// 1 or 2 at head_dim 512); K/V of type kv_dtype (bf16, fp16 or fp32).
hipError_t launch_valu(const DecodeParams& p, int head_dim, int kv_dtype, int qw, bool split, hipStream_t s);
bool valu_supported(int head_dim, int qw, int kv_dtype);

// Matrix-core decode kernel (16 query rows per MFMA tile); bf16 or fp16 K/V;
// head_dim 128, 256 or 512 (the balanced schedule: 128 or 256).
hipError_t launch_mfma(const DecodeParams& p, int head_dim, int kv_dtype, int qw, bool split, hipStream_t s);
bool mfma_supported(int head_dim, int qw, int kv_dtype);
bool mfma_lean_supported(int head_dim, int qw, int kv_dtype);
// Several queries per sequence: head_dim 128, 256 or 512, bf16 or fp16 K/V;
// the staged kernel at 128 and 256; the per-block kernel's dynamic LDS (page
// ids and block prefix sums) at most prefill_dynamic_lds_limit bytes.
bool prefill_supported(int head_dim, int kv_dtype);
bool prefill_staged_supported(int head_dim);
size_t prefill_dynamic_lds_limit(int head_dim);

// Matrix-core decode over a balanced schedule (the sequence-major list of
// (sequence, query block, 16-token tile) cut into one static unit per
// workgroup and dynamic units taken from a counter), followed by the merge
// of the units' partials.
hipError_t launch_mfma_lean(const DecodeParams& p, int head_dim, int kv_dtype, int n_wg, hipStream_t s);
constexpr int kLeanTokensPerFill = 4096;     // tokens whose page ids one LDS fill holds
// Page-id LDS entries of the balanced schedule: a run of kLeanTokensPerFill
// tokens spans at most ceil(kLeanTokensPerFill / P) + 1 pages.
inline int lean_page_slots(int page_size) { return kLeanTokensPerFill / page_size + 2; }
// Units of the balanced schedule: static units cover kLeanStaticNum /
// kLeanStaticDen of the work, the rest is cut into at most kLeanDynPerWg
// dynamic units per workgroup of at least kLeanMinUnit tiles.
constexpr int kLeanStaticNum = 4, kLeanStaticDen = 5;
constexpr int kLeanDynPerWg = 6;
constexpr int kLeanMinUnit = 16;
// Below this many tiles per workgroup the static units cover all the work.
constexpr int kLeanDynMinPerWg = 256;
// Workspace: its first kWorkspaceZeroBytes are counters that are zero
// between calls (every call leaves them so): the balanced schedule's two at
// byte 0, then one arrival counter per (sequence, query block) group for
// partitions merged inside the decode kernel, at most kFuseMaxGroups.
constexpr int kLeanCounterBytes = 256;
constexpr int kWorkspaceZeroBytes = 65536;
constexpr int kFuseCounterOffset = kLeanCounterBytes;
constexpr int kFuseMaxGroups = (kWorkspaceZeroBytes - kFuseCounterOffset) / 4;

// Several queries per sequence (MFMA, 16-column query blocks), followed by
// the per-row merge when split.
hipError_t launch_prefill(const DecodeParams& p, int head_dim, int kv_dtype, bool split, hipStream_t s);
// The same with kStagedWaves query blocks per workgroup sharing K/V stages in
// LDS (no split); p.n_slots counts workgroup slots.  Stage buffers: two at
// head_dim 128 (64 KiB, so two workgroups share a CU), four at 256 (the
// register file allows one workgroup per CU there; measured on the
// chunked-prefill workload).
constexpr int kStagedWaves = 8;
constexpr int kStagedBuffers128 = 2;
constexpr int kStagedBuffers256 = 4;
hipError_t launch_prefill_staged(const DecodeParams& p, int head_dim, int kv_dtype, hipStream_t s);

// KV-cache append (one workgroup per sequence).
hipError_t launch_append(const AppendParams& a, hipStream_t s);

// Fitted partitions (matrix-core decode): the partition size is chosen per
// call on the device from the sequence lengths, so that the live partitions
// fill a given number of workgroups; every workgroup reads all lengths, so
// the batch is bounded.
constexpr int kFitMaxBatch = 256;
constexpr int kFitMaxTokens = 1 << 24;       // block-table capacity MaxBlk * P below this

// Log-sum-exp merge of split partials into bf16 output.
hipError_t launch_merge(const DecodeParams& p, int head_dim, hipStream_t s);

}  // namespace pa
