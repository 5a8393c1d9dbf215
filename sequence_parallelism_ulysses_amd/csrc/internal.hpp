// Internal launcher interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by api.cpp and only
// enqueues work on `stream`; it returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ulysses.h"

namespace uly {

#define ULY_PERMUTE_MAX_SEGMENTS 3

// Byte-level description of one pack/unpack call: nseg segments (one for a
// single tensor; Q, K, V of a fused QKV tensor or of three tensors), each
// moved between its own shards and its own packed tensor.
struct PermuteDesc {
  int P;
  int64_t T;             // tokens per shard
  int nseg;              // 1 .. ULY_PERMUTE_MAX_SEGMENTS
  int64_t row_bytes[ULY_PERMUTE_MAX_SEGMENTS];    // bytes of one shard token of segment s (all its heads)
  int64_t seg_bytes[ULY_PERMUTE_MAX_SEGMENTS];    // hh * D * elem of segment s
  int64_t head_offset[ULY_PERMUTE_MAX_SEGMENTS];  // byte offset of segment s in a shard token
};

// shards[s]: the P shard pointers of segment s; out / in: nseg packed tensors.
hipError_t launch_pack(const void* const* const* shards, void* const* out, const PermuteDesc& d,
                       hipStream_t stream);
hipError_t launch_unpack(const void* const* in, void* const* const* shards, const PermuteDesc& d,
                         hipStream_t stream);

struct AttnDesc {
  int64_t N;
  int hq, hk, D;
  uly_dtype dt;
  const int32_t* cu;     // device, or nullptr
  int ndocs;             // number of documents (1 when cu is nullptr)
  float scale;
  int causal;            // 1: key j visible to query i iff j <= i (and same document); 0: same document
  int accumulate;        // backward only: add to dq, dk, dv (fp32 gradients) instead of overwriting
  int splits;            // backward only: workgroups per dK/dV key block (0: the default)
};

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           const AttnDesc& d, hipStream_t stream);

// attn_fwd reading Q, K, V in place from P sequence-sharded tensors (bf16,
// T a multiple of 64); d describes the head group (N = P*T, hq, hk).
hipError_t launch_attn_fwd_from_shards(const void* const* q_shards, const void* const* k_shards,
                                       const void* const* v_shards, int P, int64_t T, int Hq, int Hkv, int group,
                                       void* o, float* lse, const AttnDesc& d, hipStream_t stream);

// o = sum_c exp(lse_c - lse) o_c, lse = log sum_c exp(lse_c), per (row, head).
hipError_t launch_attn_merge(const void* const* o_parts, const float* const* lse_parts, int nparts, int64_t N,
                             int hq, int D, uly_dtype dt, void* o, float* lse, hipStream_t stream);

// Workspace of the backward (workspace.cpp): per-row delta and lse*log2(e)
// (float32 [hq][N] each); for bf16 inputs the maxima the fp16 operand
// scales derive from (kBwdMaxima uint32 slots) and the fp16 copies of q,
// dout ([N][hq][D]) and k, v ([N][hk][D]); the float32 partial dK/dV sums of
// the workgroups sharing a key block when there are several.
constexpr int kBwdMaxima = 384;
struct BwdWorkspace {
  size_t delta, lse2, absmax, q16, do16, k16, v16, part, total;
};
int bwd_dkdv_splits(const AttnDesc& d);
BwdWorkspace bwd_workspace_layout(const AttnDesc& d);
size_t bwd_workspace_bytes(const AttnDesc& d);
// attn_bwd with the library's own static device buffer as workspace (one
// workgroup per dK/dV key block, so that no partial sums need space).
// Returns hipErrorInvalidValue without launching when the sizes need more
// than kNoAllocScratchBytes (*need is then set).
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t launch_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   const AttnDesc& d, hipStream_t stream, size_t* need);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* workspace, const AttnDesc& d, uly_dtype grad_dt, hipStream_t stream);

}  // namespace uly
