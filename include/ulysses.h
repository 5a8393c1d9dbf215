/*
 * ulysses.h -- C ABI for one GPU's share of Ulysses sequence parallelism on
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("Ulysses Sequence Parallelism: Training with Million-Token
 * Contexts", Hugging Face blog, and "Snowflake's Ulysses trick trains
 * transformers on million-token contexts across GPUs", second paragraph):
 * every GPU holds a contiguous block of the sequence; an all-to-all regroups
 * the data so that each GPU holds the whole sequence for a subset of the
 * attention heads; each GPU runs ordinary attention on its heads (heads are
 * independent); a second all-to-all restores the sequence sharding. This
 * library implements the per-GPU pieces of that path:
 *
 *   ulysses_pack     sequence-sharded -> head-sharded layout for one head group
 *   attn_fwd         causal or document-masked (optionally packed-document) GQA
 *                    attention forward
 *   attn_fwd_from_shards  the same, reading sequence-sharded Q/K/V in place
 *   attn_merge       combine attention results over disjoint key chunks (LSE merge)
 *   attn_bwd         its backward (dQ, dK, dV) with logsumexp recompute
 *   attn_bwd_ex      the same with float32 gradients from bf16 inputs
 *   attn_bwd_accumulate  the same, adding to the gradients (chunked attention)
 *   attn_bwd_noalloc the same without a workspace argument (a static buffer)
 *   ulysses_unpack   head-sharded -> sequence-sharded (the inverse of pack)
 *   ulysses_pack_heads / ulysses_unpack_heads
 *                    the same for any run of heads (replicated kv heads)
 *   ulysses_pack_multi / ulysses_unpack_multi
 *                    the same for up to three tensors in one launch
 *   ulysses_pack_qkv / ulysses_unpack_qkv
 *                    the same for a fused QKV projection output, one launch
 *
 * Notation: P ranks; T tokens per rank; N = P*T; H heads in a shard tensor;
 * a head group g owns the hh = H/P contiguous heads [g*hh, (g+1)*hh).
 * hq / hk = query / key-value heads of the group; G = hq/hk q heads share one
 * kv head (local q head h reads kv head h / G). D = head dim (64 or 128).
 *
 * Layouts (all row-major, D contiguous, no padding):
 *   shard tensor      [T][H][D]     token-major, one per rank
 *   head-group tensor [N][hh][D]    what the all-to-all delivers
 *   lse               float32 [hq][N], natural log of the softmax denominator
 *   cu_seqlens        int32 [ndocs+1] document offsets into the N tokens
 *
 * Element types: ULY_F32 (IEEE float32) or ULY_BF16 (bfloat16 stored as its
 * 16 raw bits). The attention kernels accumulate in float32; bf16 outputs are
 * rounded to nearest-even.
 *
 * Conventions for every call:
 *   - The caller owns all memory. The library never allocates, frees or
 *     synchronises; it only enqueues kernels on `stream` (0 = null stream)
 *     and returns. A kernel fault surfaces at the caller's next synchronise.
 *   - All pointers except host_cu and the `shards` arrays themselves are
 *     device pointers and must be 16-byte aligned. Inputs and outputs must
 *     not alias.
 *   - Every argument is checked on the host before any HIP call. A failed
 *     check returns ULY_ERR_INVALID_ARG (bad value) or ULY_ERR_UNSUPPORTED
 *     (valid but not implemented), sets the thread-local message returned by
 *     uly_last_error(), and launches nothing. A failed HIP launch returns
 *     ULY_ERR_HIP with the HIP error text. Nothing is thrown across the ABI.
 */
#ifndef ULYSSES_H_
#define ULYSSES_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ULY_OK = 0,
  ULY_ERR_INVALID_ARG = 1,
  ULY_ERR_UNSUPPORTED = 2,
  ULY_ERR_HIP = 3
} uly_status;

typedef enum { ULY_F32 = 0, ULY_BF16 = 1 } uly_dtype;

/* Largest rank count a single pack/unpack call accepts (the shard pointers
 * travel as kernel arguments). */
#define ULY_MAX_P 64

/*
 * ulysses_pack -- the local half of the first all-to-all ("Snowflake's
 * Ulysses trick ...", second paragraph: afterwards each GPU holds the full
 * sequence for a subset of heads; "Ulysses Sequence Parallelism ...", the
 * "Sequence Sharding" step: rank j holds a contiguous block of tokens).
 *
 *   out[j*T + t][h][:] = shards[j][t][group*hh + h][:]   j < P, t < T, h < hh
 *
 * shards : host array of P device pointers, each to a [T][H][D] tensor (read).
 * out    : device [P*T][hh][D] (written in full).
 * P in [1, ULY_MAX_P]; T >= 1; H % P == 0; D in {64, 128}; 0 <= group < P.
 * The copy is bit-exact (NaN payloads included).
 */
uly_status ulysses_pack(const void* const* shards, int P, int64_t T, int H, int D,
                        uly_dtype dt, int group, void* out, hipStream_t stream);

/*
 * ulysses_unpack -- the local half of the second all-to-all, which reverses
 * the first and returns to sequence sharding ("Ulysses Sequence Parallelism
 * ...", "All-to-All Communication" step).
 *
 *   shards[j][t][group*hh + h][:] = in[j*T + t][h][:]
 *
 * in     : device [P*T][hh][D] (read).
 * shards : host array of P device pointers to [T][H][D] tensors; only the
 *          group's heads are written, every other head is left untouched.
 * Same preconditions as ulysses_pack; bit-exact.
 */
uly_status ulysses_unpack(const void* in, int P, int64_t T, int H, int D, uly_dtype dt,
                          int group, void* const* shards, hipStream_t stream);

/*
 * ulysses_pack_heads -- the same regrouping for any run of heads:
 *
 *   out[j*T + t][h][:] = shards[j][t][head0 + h][:]      j < P, t < T, h < nheads
 *
 * With head0 = group*H/P and nheads = H/P it is ulysses_pack. Its other use
 * is a tensor with fewer heads than ranks (Hkv < P): the pages do not cover
 * that case; here the key/value heads are then replicated, rank g (query
 * heads [g*Hq/P, (g+1)*Hq/P)) gathering the one kv head those query heads
 * read, head0 = floor(g * Hkv / P), nheads = 1 (requires P % Hkv == 0). The
 * backward's dK/dV of such a head is then a sum over the P/Hkv ranks sharing
 * it, a reduction across ranks that this library does not perform.
 * shards : host array of P device pointers to [T][H][D] tensors (read).
 * out    : device [P*T][nheads][D] (written in full).
 * P in [1, ULY_MAX_P]; T >= 1; 1 <= nheads and 0 <= head0 <= H - nheads;
 * D in {64, 128}. Bit-exact; errors as ulysses_pack.
 */
uly_status ulysses_pack_heads(const void* const* shards, int P, int64_t T, int H, int D, uly_dtype dt,
                              int head0, int nheads, void* out, hipStream_t stream);

/*
 * ulysses_unpack_heads -- the inverse of ulysses_pack_heads:
 *   shards[j][t][head0 + h][:] = in[j*T + t][h][:]
 * Every other head is left untouched. Same preconditions.
 */
uly_status ulysses_unpack_heads(const void* in, int P, int64_t T, int H, int D, uly_dtype dt, int head0,
                                int nheads, void* const* shards, hipStream_t stream);

/*
 * ulysses_pack_multi -- ulysses_pack of up to three tensors in one launch,
 * e.g. Q, K and V as their projections leave them, each sequence-sharded
 * with its own head count. For tensor i and its hh_i = H[i]/P heads:
 *
 *   outs[i][j*T + t][h][:] = shards[i*P + j][t][group*hh_i + h][:]
 *
 * ntensors in [1, 3]. shards: host array of ntensors*P device pointers,
 * tensor-major, each [T][H[i]][D]. H: host array of ntensors head counts.
 * outs: host array of ntensors device pointers, outs[i] [P*T][hh_i][D]
 * (written in full). P, T, D, dt and group are shared; each tensor must
 * satisfy the ulysses_pack preconditions. Bit-exact.
 */
uly_status ulysses_pack_multi(int ntensors, const void* const* shards, const int* H, int P, int64_t T,
                              int D, uly_dtype dt, int group, void* const* outs, hipStream_t stream);

/*
 * ulysses_unpack_multi -- ulysses_unpack of up to three tensors in one launch
 * (e.g. dQ, dK and dV back to their sequence-sharded gradients):
 *
 *   shards[i*P + j][t][group*hh_i + h][:] = ins[i][j*T + t][h][:]
 *
 * Only the group's heads are written; every other head is left untouched.
 * Arguments as ulysses_pack_multi with ins[i] the [P*T][hh_i][D] inputs.
 */
uly_status ulysses_unpack_multi(int ntensors, const void* const* ins, const int* H, int P, int64_t T,
                                int D, uly_dtype dt, int group, void* const* shards, hipStream_t stream);

/*
 * ulysses_pack_qkv -- ulysses_pack for the output of a fused QKV projection,
 * in one launch ("Snowflake's Ulysses trick ...", second paragraph: the
 * all-to-all follows each GPU's local QKV projections). The pages do not give
 * the fused layout; here a shard token holds the Hq query heads, then the Hkv
 * key heads, then the Hkv value heads, each D elements:
 *
 *   shards[j] : [T][Hq + 2*Hkv][D]   (query heads [0, Hq), key heads
 *               [Hq, Hq+Hkv), value heads [Hq+Hkv, Hq+2*Hkv))
 *   q_out[j*T + t][h][:] = shards[j][t][group*hq + h][:]             h < hq = Hq/P
 *   k_out[j*T + t][h][:] = shards[j][t][Hq + group*hk + h][:]        h < hk = Hkv/P
 *   v_out[j*T + t][h][:] = shards[j][t][Hq + Hkv + group*hk + h][:]
 *
 * q_out : device [P*T][hq][D]; k_out, v_out : device [P*T][hk][D] (written
 * in full). P in [1, ULY_MAX_P]; T >= 1; Hq % P == 0 and Hkv % P == 0;
 * D in {64, 128}; 0 <= group < P. Bit-exact; other preconditions and errors
 * as ulysses_pack.
 */
uly_status ulysses_pack_qkv(const void* const* shards, int P, int64_t T, int Hq, int Hkv, int D,
                            uly_dtype dt, int group, void* q_out, void* k_out, void* v_out,
                            hipStream_t stream);

/*
 * ulysses_unpack_qkv -- the inverse of ulysses_pack_qkv, in one launch: the
 * head-group gradients dq [P*T][hq][D], dk and dv [P*T][hk][D] go back into
 * the fused [T][Hq + 2*Hkv][D] layout of each shard (the gradient of the
 * fused projection output; the backward's mirror of the second all-to-all).
 * Only the group's heads of each section are written; every other head is
 * left untouched. Same preconditions as ulysses_pack_qkv; bit-exact.
 */
uly_status ulysses_unpack_qkv(const void* dq, const void* dk, const void* dv, int P, int64_t T, int Hq,
                              int Hkv, int D, uly_dtype dt, int group, void* const* shards,
                              hipStream_t stream);

/*
 * attn_fwd -- exact softmax attention for one head group over the full
 * sequence ("Snowflake's Ulysses trick ...", second paragraph: each GPU runs
 * standard attention on its heads; "Ulysses Sequence Parallelism ...": tiled
 * attention keeps memory linear while computing the same result).
 *
 * For local q head h (kv head h/G), query i and key j, with the mask
 * M_ij = (j <= i or causal == 0) and doc(j) == doc(i):
 *   S_ij = softmax_scale * q_i . k_j              (masked: -inf)
 *   lse_i = log sum_j exp(S_ij)                   (natural log)
 *   o_i  = sum_j exp(S_ij - lse_i) v_j
 *
 * q, o     : device [N][hq][D] of dt.   k, v : device [N][hk][D] of dt.
 * lse      : device float32 [hq][N] (written; attn_bwd reads it).
 * cu_seqlens : device int32 [ndocs+1], non-decreasing from 0 to N (empty
 *            documents allowed), or NULL for one document of N tokens. Its
 *            contents are a precondition, not checked here (see
 *            uly_check_cu_seqlens); ndocs is ignored when it is NULL.
 * causal : 1 for the causal mask the configurations use (the pages train
 *          causal language models); 0 drops the j <= i bound, so every token
 *          sees its whole document (the pages do not say; offered because
 *          a key/value chunk that lies entirely before a query chunk, as in
 *          chunked or ring-style attention, is seen this way).
 * N >= 1; hq % hk == 0; D in {64, 128}; softmax_scale finite and > 0;
 * causal in {0, 1}. ULY_F32 requires D == 64 or 128 and runs in float32
 * throughout.
 */
uly_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t N, int hq, int hk, int D, uly_dtype dt,
                    const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                    hipStream_t stream);

/*
 * attn_fwd_from_shards -- attn_fwd for head group `group` reading Q, K and V
 * in place from the sequence-sharded tensors, so that on one GPU their pack
 * disappears: the kernels' tile loads take token n of the group from shard
 * n / T, row n % T, heads [group*Hq/P, ...) and [group*Hkv/P, ...). Same
 * result, bit for bit, as ulysses_pack of Q, K and V followed by attn_fwd.
 *
 * q_shards : host array of P device pointers to [T][Hq][D]; k_shards,
 *            v_shards : likewise [T][Hkv][D].
 * o        : device [P*T][Hq/P][D] (head-group layout, as attn_fwd writes it).
 * lse      : device float32 [Hq/P][P*T].
 * Requires dt == ULY_BF16 and T % 64 == 0 (else ULY_ERR_UNSUPPORTED),
 * Hq % P == 0, Hkv % P == 0, 0 <= group < P; other arguments and errors as
 * attn_fwd with N = P*T, hq = Hq/P, hk = Hkv/P.
 */
uly_status attn_fwd_from_shards(const void* const* q_shards, const void* const* k_shards,
                                const void* const* v_shards, int P, int64_t T, int Hq, int Hkv, int D,
                                uly_dtype dt, int group, void* o, float* lse, const int32_t* cu_seqlens,
                                int ndocs, float softmax_scale, int causal, hipStream_t stream);

/*
 * attn_merge -- combine attention results computed over disjoint sets of
 * keys into the result over their union, as a ring of key/value chunks
 * produces them ("Snowflake's Ulysses trick ...", third paragraph: the
 * comparison with Ring Attention, which passes chunks around a ring). For
 * every row i and local q head h, with parts c = 0 .. nparts-1:
 *   lse[h][i] = log sum_c exp(lse_c[h][i])
 *   o[i][h][:] = sum_c exp(lse_c[h][i] - lse[h][i]) * o_c[i][h][:]
 * (fp32 arithmetic, max-shifted; o rounded to nearest even for bf16). A part
 * whose lse is -inf (no visible key) contributes nothing; if every part's is,
 * o = 0 and lse = -inf.
 *
 * o_parts   : host array of nparts device pointers to [N][hq][D] of dt, each
 *             the normalised output over its key set (as attn_fwd writes it).
 * lse_parts : host array of nparts device pointers to float32 [hq][N].
 * o         : device [N][hq][D] of dt; lse : device float32 [hq][N]; neither
 *             may alias a part.
 * nparts in [1, ULY_MAX_P]; N in [1, 2^30]; hq in [1, 1024]; D in {64, 128}.
 */
uly_status attn_merge(const void* const* o_parts, const float* const* lse_parts, int nparts, int64_t N,
                      int hq, int D, uly_dtype dt, void* o, float* lse, hipStream_t stream);

/*
 * attn_bwd_workspace_size -- bytes of device workspace attn_bwd (and
 * attn_bwd_ex, attn_bwd_accumulate) needs for these sizes: the per-row
 * delta_i = dO_i . O_i and lse_i * log2(e) (float32 [hq][N] each); for
 * bf16 inputs also six float32 maxima and the power-of-two-scaled fp16
 * copies of q, dout, k and v that the products read (2 x N x (hq + hk) x D
 * halves); and the float32 partial dK/dV sums of the workgroups that share
 * a key block (2 x 4 x N x hk x D floats). Each part starts on a 256-byte
 * boundary.
 */
uly_status attn_bwd_workspace_size(int64_t N, int hq, int hk, int D, uly_dtype dt,
                                   size_t* bytes);

/*
 * attn_bwd -- the backward of attn_fwd for one head group. The pages train
 * with this path ("Ulysses Sequence Parallelism: Training with Million-Token
 * Contexts", opening paragraph; "Snowflake's Ulysses trick ...", fourth
 * paragraph: fine-tuning through the same attention handler), so each GPU
 * also computes the gradients of the attention over its heads (second
 * paragraph of the same page: heads are independent). With the softmax
 * probabilities recomputed from lse, the gradients of L = sum(dout * o) are
 *   delta_i = dout_i . o_i
 *   P_ij  = exp(S_ij - lse_i)            dP_ij = dout_i . v_j
 *   dS_ij = P_ij (dP_ij - delta_i)
 *   dq_i  = scale * sum_j dS_ij k_j
 *   dk_j  = scale * sum_{h in group} sum_i dS_ij q_i
 *   dv_j  = sum_{h in group} sum_i P_ij dout_i
 * q, o, dout : device [N][hq][D] of dt; k, v : device [N][hk][D] of dt;
 * lse : device float32 [hq][N] from attn_fwd with the same inputs.
 * dq : device [N][hq][D], dk, dv : device [N][hk][D], all of dt (bf16
 * gradients are the float32 results rounded to nearest even). They are
 * overwritten; dk/dv hold the sum over the G q heads of each kv head.
 * workspace: device memory of at least attn_bwd_workspace_size() bytes,
 * 16-byte aligned, owned by the caller, contents ignored on entry.
 * causal must match the attn_fwd call that produced o and lse. Other
 * preconditions and errors as attn_fwd. Results are bitwise repeatable (no
 * atomic adds: every sum has a fixed order).
 */
uly_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    int64_t N, int hq, int hk, int D, uly_dtype dt,
                    const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_bwd_ex -- attn_bwd with the gradient type appended to its argument
 * list: grad_dt is dt, or ULY_F32 for float32 gradients from bf16 inputs
 * (the same computation, stored before the final rounding). Everything else
 * as attn_bwd (same workspace size). Errors: ULY_ERR_INVALID_ARG for an
 * unknown grad_dt, ULY_ERR_UNSUPPORTED for grad_dt other than dt or ULY_F32.
 */
uly_status attn_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       int64_t N, int hq, int hk, int D, uly_dtype dt,
                       const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       uly_dtype grad_dt);

/*
 * attn_bwd_accumulate -- attn_bwd that adds its gradients to dq, dk and dv
 * instead of overwriting them. This is what the backward of attention over
 * key/value chunks needs (the chunks of Ring Attention, "Snowflake's Ulysses
 * trick ...", third paragraph): with o and lse the merged results over all
 * chunks (attn_merge), one call per (query chunk, key chunk) pair adds that
 * pair's share to the query chunk's dq and the key chunk's dk and dv, and
 * the sums equal the gradients of attention over the union.
 * Same arguments and preconditions as attn_bwd, except that dq, dk and dv
 * are float32 whatever dt is (accumulating in bf16 would round at every
 * call) and must hold the values to add to.
 */
uly_status attn_bwd_accumulate(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               int64_t N, int hq, int hk, int D, uly_dtype dt,
                               const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments as attn_bwd without the workspace; the
 * library's own static device buffer of ULY_NOALLOC_SCRATCH_BYTES serves as
 * workspace (each GPU the library runs on holds its copy until the process
 * ends), and each dK/dV key block is done by one workgroup (no partial sums),
 * so dq is bitwise the same as attn_bwd's and dk/dv differ from it only in
 * the order of their float32 sums. The call allocates nothing and frees
 * nothing. Sizes whose workspace exceeds the buffer return
 * ULY_ERR_UNSUPPORTED (bf16, 4 q heads on 1 kv head, D = 128: up to 51780
 * tokens); a stream that does not belong to the current device returns
 * ULY_ERR_INVALID_ARG. Every call on one GPU uses the same buffer: calls that
 * overlap in time on one GPU (on several streams, or from several host
 * threads) race and give wrong results. Other preconditions and errors as
 * attn_bwd.
 */
#define ULY_NOALLOC_SCRATCH_BYTES (128u << 20)
uly_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            int64_t N, int hq, int hk, int D, uly_dtype dt,
                            const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                            hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none).
 * Never NULL; valid until the next call on the same thread. */
const char* uly_last_error(void);

/* Host-side check of document offsets: host_cu[0] == 0, non-decreasing,
 * host_cu[ndocs] == N, ndocs >= 1. Returns ULY_OK or ULY_ERR_INVALID_ARG. */
uly_status uly_check_cu_seqlens(const int32_t* host_cu, int ndocs, int64_t N);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H_ */
