// C ABI entry points: host-side argument checks, then one launcher call.
// Every check runs before any HIP call, so invalid arguments are reported
// without touching the GPU (and can be tested on a machine without one).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "internal.hpp"

namespace {

thread_local std::string g_last_error;

uly_status fail(uly_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

uly_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ULY_OK;
  return fail(ULY_ERR_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(uly_dtype dt) { return dt == ULY_BF16 ? 2 : 4; }

bool valid_dtype(int dt) { return dt == ULY_F32 || dt == ULY_BF16; }

#define CHECK(cond, status, ...)              \
  do {                                        \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

uly_status check_permute(const char* fn, int P, int64_t T, int H, int D, int dt, int group,
                         uly::PermuteDesc* out) {
  CHECK(P >= 1 && P <= ULY_MAX_P, ULY_ERR_INVALID_ARG, "%s: P=%d must be in [1, %d]", fn, P, ULY_MAX_P);
  CHECK(T >= 1, ULY_ERR_INVALID_ARG, "%s: T=%lld must be >= 1", fn, (long long)T);
  CHECK(H >= 1 && H % P == 0, ULY_ERR_INVALID_ARG, "%s: H=%d must be a positive multiple of P=%d", fn, H, P);
  CHECK(D == 64 || D == 128, ULY_ERR_INVALID_ARG, "%s: D=%d must be 64 or 128", fn, D);
  CHECK(valid_dtype(dt), ULY_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dt);
  CHECK(group >= 0 && group < P, ULY_ERR_INVALID_ARG, "%s: group=%d must be in [0, P=%d)", fn, group, P);
  const int64_t e = elem_bytes(static_cast<uly_dtype>(dt));
  const int64_t hh = H / P;
  out->P = P;
  out->T = T;
  out->row_bytes[0] = H * D * e;
  out->nseg = 1;
  out->seg_bytes[0] = hh * D * e;
  out->head_offset[0] = group * hh * D * e;
  CHECK(T * (out->seg_bytes[0] / 16) < (int64_t(1) << 31), ULY_ERR_UNSUPPORTED,
        "%s: one shard's head group (%lld bytes) exceeds 32 GiB", fn, (long long)(T * out->seg_bytes[0]));
  return ULY_OK;
}

// Any run of heads [head0, head0 + nheads) of every shard token.
uly_status check_heads(const char* fn, int P, int64_t T, int H, int D, int dt, int head0, int nheads,
                       uly::PermuteDesc* out) {
  CHECK(P >= 1 && P <= ULY_MAX_P, ULY_ERR_INVALID_ARG, "%s: P=%d must be in [1, %d]", fn, P, ULY_MAX_P);
  CHECK(T >= 1, ULY_ERR_INVALID_ARG, "%s: T=%lld must be >= 1", fn, (long long)T);
  CHECK(H >= 1 && H <= (1 << 20), ULY_ERR_INVALID_ARG, "%s: H=%d must be in [1, 2^20]", fn, H);
  CHECK(D == 64 || D == 128, ULY_ERR_INVALID_ARG, "%s: D=%d must be 64 or 128", fn, D);
  CHECK(valid_dtype(dt), ULY_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dt);
  CHECK(nheads >= 1 && head0 >= 0 && head0 <= H - nheads, ULY_ERR_INVALID_ARG,
        "%s: heads [%d, %d + %d) must lie in [0, H=%d)", fn, head0, head0, nheads, H);
  const int64_t e = elem_bytes(static_cast<uly_dtype>(dt));
  out->P = P;
  out->T = T;
  out->nseg = 1;
  out->row_bytes[0] = int64_t(H) * D * e;
  out->seg_bytes[0] = int64_t(nheads) * D * e;
  out->head_offset[0] = int64_t(head0) * D * e;
  CHECK(T * (out->seg_bytes[0] / 16) < (int64_t(1) << 31), ULY_ERR_UNSUPPORTED,
        "%s: one shard's heads (%lld bytes) exceed 32 GiB", fn, (long long)(T * out->seg_bytes[0]));
  return ULY_OK;
}

// A fused QKV shard token holds Hq query heads, then Hkv key heads, then Hkv
// value heads; the group's slice of each section is one segment.
uly_status check_permute_qkv(const char* fn, int P, int64_t T, int Hq, int Hkv, int D, int dt, int group,
                             uly::PermuteDesc* out) {
  CHECK(P >= 1 && P <= ULY_MAX_P, ULY_ERR_INVALID_ARG, "%s: P=%d must be in [1, %d]", fn, P, ULY_MAX_P);
  CHECK(T >= 1, ULY_ERR_INVALID_ARG, "%s: T=%lld must be >= 1", fn, (long long)T);
  CHECK(Hq >= 1 && Hq % P == 0, ULY_ERR_INVALID_ARG, "%s: Hq=%d must be a positive multiple of P=%d", fn, Hq, P);
  CHECK(Hkv >= 1 && Hkv % P == 0, ULY_ERR_INVALID_ARG, "%s: Hkv=%d must be a positive multiple of P=%d", fn, Hkv, P);
  CHECK(Hq <= (1 << 20) && Hkv <= (1 << 20), ULY_ERR_INVALID_ARG, "%s: Hq=%d, Hkv=%d too large", fn, Hq, Hkv);
  CHECK(D == 64 || D == 128, ULY_ERR_INVALID_ARG, "%s: D=%d must be 64 or 128", fn, D);
  CHECK(valid_dtype(dt), ULY_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dt);
  CHECK(group >= 0 && group < P, ULY_ERR_INVALID_ARG, "%s: group=%d must be in [0, P=%d)", fn, group, P);
  const int64_t e = elem_bytes(static_cast<uly_dtype>(dt));
  const int64_t hq = Hq / P, hk = Hkv / P;
  out->P = P;
  out->T = T;
  out->row_bytes[0] = out->row_bytes[1] = out->row_bytes[2] = int64_t(Hq + 2 * Hkv) * D * e;
  out->nseg = 3;
  out->seg_bytes[0] = hq * D * e;
  out->seg_bytes[1] = out->seg_bytes[2] = hk * D * e;
  out->head_offset[0] = group * hq * D * e;
  out->head_offset[1] = (int64_t(Hq) + group * hk) * D * e;
  out->head_offset[2] = (int64_t(Hq) + Hkv + group * hk) * D * e;
  for (int sg = 0; sg < 3; ++sg)
    CHECK(T * (out->seg_bytes[sg] / 16) < (int64_t(1) << 31), ULY_ERR_UNSUPPORTED,
          "%s: one shard's head group (%lld bytes) exceeds 32 GiB", fn, (long long)(T * out->seg_bytes[sg]));
  return ULY_OK;
}

uly_status check_attn(const char* fn, int64_t N, int hq, int hk, int D, int dt,
                      const int32_t* cu, int ndocs, float scale, int causal, uly::AttnDesc* d) {
  CHECK(N >= 1 && N <= (int64_t(1) << 30), ULY_ERR_INVALID_ARG, "%s: N=%lld must be in [1, 2^30]", fn, (long long)N);
  CHECK(hq >= 1 && hk >= 1 && hq <= 1024, ULY_ERR_INVALID_ARG, "%s: hq=%d, hk=%d must be positive (hq <= 1024)", fn, hq, hk);
  CHECK(hq % hk == 0, ULY_ERR_INVALID_ARG, "%s: hq=%d must be a multiple of hk=%d", fn, hq, hk);
  CHECK(D == 64 || D == 128, ULY_ERR_INVALID_ARG, "%s: D=%d must be 64 or 128", fn, D);
  CHECK(valid_dtype(dt), ULY_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dt);
  CHECK(std::isfinite(scale) && scale > 0.f, ULY_ERR_INVALID_ARG, "%s: softmax_scale=%g must be finite and > 0", fn, (double)scale);
  CHECK(causal == 0 || causal == 1, ULY_ERR_INVALID_ARG, "%s: causal=%d must be 0 or 1", fn, causal);
  CHECK(cu == nullptr || ndocs >= 1, ULY_ERR_INVALID_ARG, "%s: ndocs=%d must be >= 1 with cu_seqlens", fn, ndocs);
  CHECK(cu == nullptr || (reinterpret_cast<uintptr_t>(cu) & 3u) == 0, ULY_ERR_INVALID_ARG,
        "%s: cu_seqlens must be 4-byte aligned", fn);
  CHECK(cu == nullptr || ndocs <= (1 << 30), ULY_ERR_INVALID_ARG, "%s: ndocs=%d too large", fn, ndocs);
  d->N = N;
  d->hq = hq;
  d->hk = hk;
  d->D = D;
  d->dt = static_cast<uly_dtype>(dt);
  d->cu = cu;
  d->ndocs = cu ? ndocs : 1;
  d->scale = scale;
  d->causal = causal;
  d->accumulate = 0;
  d->splits = 0;
  return ULY_OK;
}

}  // namespace

extern "C" {

const char* uly_last_error(void) { return g_last_error.c_str(); }

uly_status uly_check_cu_seqlens(const int32_t* host_cu, int ndocs, int64_t N) {
  CHECK(host_cu != nullptr, ULY_ERR_INVALID_ARG, "uly_check_cu_seqlens: host_cu is NULL");
  CHECK(ndocs >= 1, ULY_ERR_INVALID_ARG, "uly_check_cu_seqlens: ndocs=%d must be >= 1", ndocs);
  CHECK(host_cu[0] == 0, ULY_ERR_INVALID_ARG, "uly_check_cu_seqlens: cu_seqlens[0]=%d must be 0", host_cu[0]);
  for (int i = 0; i < ndocs; ++i)
    CHECK(host_cu[i + 1] >= host_cu[i], ULY_ERR_INVALID_ARG,
          "uly_check_cu_seqlens: offsets decrease at %d (%d > %d)", i, host_cu[i], host_cu[i + 1]);
  CHECK(host_cu[ndocs] == N, ULY_ERR_INVALID_ARG, "uly_check_cu_seqlens: cu_seqlens[%d]=%d must equal N=%lld",
        ndocs, host_cu[ndocs], (long long)N);
  return ULY_OK;
}

uly_status ulysses_pack(const void* const* shards, int P, int64_t T, int H, int D, uly_dtype dt,
                        int group, void* out, hipStream_t stream) {
  uly::PermuteDesc d;
  uly_status s = check_permute("ulysses_pack", P, T, H, D, dt, group, &d);
  if (s != ULY_OK) return s;
  CHECK(shards != nullptr, ULY_ERR_INVALID_ARG, "ulysses_pack: shards is NULL");
  CHECK(out != nullptr && aligned16(out), ULY_ERR_INVALID_ARG, "ulysses_pack: out is NULL or not 16-byte aligned");
  for (int j = 0; j < P; ++j)
    CHECK(shards[j] != nullptr && aligned16(shards[j]), ULY_ERR_INVALID_ARG,
          "ulysses_pack: shards[%d] is NULL or not 16-byte aligned", j);
  void* const outs[1] = {out};
  const void* const* sh[1] = {shards};
  return from_hip(uly::launch_pack(sh, outs, d, stream), "ulysses_pack");
}

uly_status ulysses_unpack(const void* in, int P, int64_t T, int H, int D, uly_dtype dt, int group,
                          void* const* shards, hipStream_t stream) {
  uly::PermuteDesc d;
  uly_status s = check_permute("ulysses_unpack", P, T, H, D, dt, group, &d);
  if (s != ULY_OK) return s;
  CHECK(shards != nullptr, ULY_ERR_INVALID_ARG, "ulysses_unpack: shards is NULL");
  CHECK(in != nullptr && aligned16(in), ULY_ERR_INVALID_ARG, "ulysses_unpack: in is NULL or not 16-byte aligned");
  for (int j = 0; j < P; ++j)
    CHECK(shards[j] != nullptr && aligned16(shards[j]), ULY_ERR_INVALID_ARG,
          "ulysses_unpack: shards[%d] is NULL or not 16-byte aligned", j);
  const void* const ins[1] = {in};
  void* const* sh[1] = {shards};
  return from_hip(uly::launch_unpack(ins, sh, d, stream), "ulysses_unpack");
}

uly_status ulysses_pack_heads(const void* const* shards, int P, int64_t T, int H, int D, uly_dtype dt, int head0,
                              int nheads, void* out, hipStream_t stream) {
  uly::PermuteDesc d;
  uly_status s = check_heads("ulysses_pack_heads", P, T, H, D, dt, head0, nheads, &d);
  if (s != ULY_OK) return s;
  CHECK(shards != nullptr, ULY_ERR_INVALID_ARG, "ulysses_pack_heads: shards is NULL");
  CHECK(out != nullptr && aligned16(out), ULY_ERR_INVALID_ARG,
        "ulysses_pack_heads: out is NULL or not 16-byte aligned");
  for (int j = 0; j < P; ++j)
    CHECK(shards[j] != nullptr && aligned16(shards[j]), ULY_ERR_INVALID_ARG,
          "ulysses_pack_heads: shards[%d] is NULL or not 16-byte aligned", j);
  void* const outs[1] = {out};
  const void* const* sh[1] = {shards};
  return from_hip(uly::launch_pack(sh, outs, d, stream), "ulysses_pack_heads");
}

uly_status ulysses_unpack_heads(const void* in, int P, int64_t T, int H, int D, uly_dtype dt, int head0, int nheads,
                                void* const* shards, hipStream_t stream) {
  uly::PermuteDesc d;
  uly_status s = check_heads("ulysses_unpack_heads", P, T, H, D, dt, head0, nheads, &d);
  if (s != ULY_OK) return s;
  CHECK(shards != nullptr, ULY_ERR_INVALID_ARG, "ulysses_unpack_heads: shards is NULL");
  CHECK(in != nullptr && aligned16(in), ULY_ERR_INVALID_ARG,
        "ulysses_unpack_heads: in is NULL or not 16-byte aligned");
  for (int j = 0; j < P; ++j)
    CHECK(shards[j] != nullptr && aligned16(shards[j]), ULY_ERR_INVALID_ARG,
          "ulysses_unpack_heads: shards[%d] is NULL or not 16-byte aligned", j);
  const void* const ins[1] = {in};
  void* const* sh[1] = {shards};
  return from_hip(uly::launch_unpack(ins, sh, d, stream), "ulysses_unpack_heads");
}

uly_status ulysses_pack_qkv(const void* const* shards, int P, int64_t T, int Hq, int Hkv, int D,
                            uly_dtype dt, int group, void* q_out, void* k_out, void* v_out,
                            hipStream_t stream) {
  uly::PermuteDesc d;
  uly_status s = check_permute_qkv("ulysses_pack_qkv", P, T, Hq, Hkv, D, dt, group, &d);
  if (s != ULY_OK) return s;
  CHECK(shards != nullptr, ULY_ERR_INVALID_ARG, "ulysses_pack_qkv: shards is NULL");
  void* const outs[3] = {q_out, k_out, v_out};
  const char* names[3] = {"q_out", "k_out", "v_out"};
  for (int i = 0; i < 3; ++i)
    CHECK(outs[i] != nullptr && aligned16(outs[i]), ULY_ERR_INVALID_ARG,
          "ulysses_pack_qkv: %s is NULL or not 16-byte aligned", names[i]);
  for (int j = 0; j < P; ++j)
    CHECK(shards[j] != nullptr && aligned16(shards[j]), ULY_ERR_INVALID_ARG,
          "ulysses_pack_qkv: shards[%d] is NULL or not 16-byte aligned", j);
  const void* const* sh[3] = {shards, shards, shards};
  return from_hip(uly::launch_pack(sh, outs, d, stream), "ulysses_pack_qkv");
}

uly_status ulysses_unpack_qkv(const void* dq, const void* dk, const void* dv, int P, int64_t T, int Hq,
                              int Hkv, int D, uly_dtype dt, int group, void* const* shards,
                              hipStream_t stream) {
  uly::PermuteDesc d;
  uly_status s = check_permute_qkv("ulysses_unpack_qkv", P, T, Hq, Hkv, D, dt, group, &d);
  if (s != ULY_OK) return s;
  CHECK(shards != nullptr, ULY_ERR_INVALID_ARG, "ulysses_unpack_qkv: shards is NULL");
  const void* const ins[3] = {dq, dk, dv};
  const char* names[3] = {"dq", "dk", "dv"};
  for (int i = 0; i < 3; ++i)
    CHECK(ins[i] != nullptr && aligned16(ins[i]), ULY_ERR_INVALID_ARG,
          "ulysses_unpack_qkv: %s is NULL or not 16-byte aligned", names[i]);
  for (int j = 0; j < P; ++j)
    CHECK(shards[j] != nullptr && aligned16(shards[j]), ULY_ERR_INVALID_ARG,
          "ulysses_unpack_qkv: shards[%d] is NULL or not 16-byte aligned", j);
  void* const* sh[3] = {shards, shards, shards};
  return from_hip(uly::launch_unpack(ins, sh, d, stream), "ulysses_unpack_qkv");
}

}  // extern "C"

namespace {

// Several tensors, each with its own shards and head count, in one launch.
uly_status check_permute_multi(const char* fn, int ntensors, const int* H, int P, int64_t T, int D, int dt,
                               int group, uly::PermuteDesc* out) {
  CHECK(ntensors >= 1 && ntensors <= ULY_PERMUTE_MAX_SEGMENTS, ULY_ERR_INVALID_ARG,
        "%s: ntensors=%d must be in [1, %d]", fn, ntensors, ULY_PERMUTE_MAX_SEGMENTS);
  CHECK(H != nullptr, ULY_ERR_INVALID_ARG, "%s: H is NULL", fn);
  for (int i = 0; i < ntensors; ++i) {
    uly::PermuteDesc one;
    char name[64];
    snprintf(name, sizeof name, "%s (tensor %d)", fn, i);
    uly_status s = check_permute(name, P, T, H[i], D, dt, group, &one);
    if (s != ULY_OK) return s;
    out->row_bytes[i] = one.row_bytes[0];
    out->seg_bytes[i] = one.seg_bytes[0];
    out->head_offset[i] = one.head_offset[0];
  }
  out->P = P;
  out->T = T;
  out->nseg = ntensors;
  return ULY_OK;
}

}  // namespace

extern "C" {

uly_status ulysses_pack_multi(int ntensors, const void* const* shards, const int* H, int P, int64_t T, int D,
                              uly_dtype dt, int group, void* const* outs, hipStream_t stream) {
  uly::PermuteDesc d;
  uly_status s = check_permute_multi("ulysses_pack_multi", ntensors, H, P, T, D, dt, group, &d);
  if (s != ULY_OK) return s;
  CHECK(shards != nullptr && outs != nullptr, ULY_ERR_INVALID_ARG, "ulysses_pack_multi: shards or outs is NULL");
  const void* const* sh[ULY_PERMUTE_MAX_SEGMENTS] = {};
  for (int i = 0; i < ntensors; ++i) {
    CHECK(outs[i] != nullptr && aligned16(outs[i]), ULY_ERR_INVALID_ARG,
          "ulysses_pack_multi: outs[%d] is NULL or not 16-byte aligned", i);
    for (int j = 0; j < P; ++j)
      CHECK(shards[i * P + j] != nullptr && aligned16(shards[i * P + j]), ULY_ERR_INVALID_ARG,
            "ulysses_pack_multi: shards[%d] is NULL or not 16-byte aligned", i * P + j);
    sh[i] = shards + i * P;
  }
  return from_hip(uly::launch_pack(sh, outs, d, stream), "ulysses_pack_multi");
}

uly_status ulysses_unpack_multi(int ntensors, const void* const* ins, const int* H, int P, int64_t T, int D,
                                uly_dtype dt, int group, void* const* shards, hipStream_t stream) {
  uly::PermuteDesc d;
  uly_status s = check_permute_multi("ulysses_unpack_multi", ntensors, H, P, T, D, dt, group, &d);
  if (s != ULY_OK) return s;
  CHECK(shards != nullptr && ins != nullptr, ULY_ERR_INVALID_ARG, "ulysses_unpack_multi: shards or ins is NULL");
  void* const* sh[ULY_PERMUTE_MAX_SEGMENTS] = {};
  for (int i = 0; i < ntensors; ++i) {
    CHECK(ins[i] != nullptr && aligned16(ins[i]), ULY_ERR_INVALID_ARG,
          "ulysses_unpack_multi: ins[%d] is NULL or not 16-byte aligned", i);
    for (int j = 0; j < P; ++j)
      CHECK(shards[i * P + j] != nullptr && aligned16(shards[i * P + j]), ULY_ERR_INVALID_ARG,
            "ulysses_unpack_multi: shards[%d] is NULL or not 16-byte aligned", i * P + j);
    sh[i] = shards + i * P;
  }
  return from_hip(uly::launch_unpack(ins, sh, d, stream), "ulysses_unpack_multi");
}

uly_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N,
                    int hq, int hk, int D, uly_dtype dt, const int32_t* cu_seqlens, int ndocs,
                    float softmax_scale, int causal, hipStream_t stream) {
  uly::AttnDesc d;
  uly_status s = check_attn("attn_fwd", N, hq, hk, D, dt, cu_seqlens, ndocs, softmax_scale, causal, &d);
  if (s != ULY_OK) return s;
  const void* ptrs[] = {q, k, v, o, lse};
  const char* names[] = {"q", "k", "v", "o", "lse"};
  for (int i = 0; i < 5; ++i)
    CHECK(ptrs[i] != nullptr && aligned16(ptrs[i]), ULY_ERR_INVALID_ARG,
          "attn_fwd: %s is NULL or not 16-byte aligned", names[i]);
  return from_hip(uly::launch_attn_fwd(q, k, v, o, lse, d, stream), "attn_fwd");
}

uly_status attn_fwd_from_shards(const void* const* q_shards, const void* const* k_shards,
                                const void* const* v_shards, int P, int64_t T, int Hq, int Hkv, int D, uly_dtype dt,
                                int group, void* o, float* lse, const int32_t* cu_seqlens, int ndocs,
                                float softmax_scale, int causal, hipStream_t stream) {
  const char* fn = "attn_fwd_from_shards";
  CHECK(P >= 1 && P <= ULY_MAX_P, ULY_ERR_INVALID_ARG, "%s: P=%d must be in [1, %d]", fn, P, ULY_MAX_P);
  CHECK(T >= 1 && T <= (int64_t(1) << 30), ULY_ERR_INVALID_ARG, "%s: T=%lld must be in [1, 2^30]", fn, (long long)T);
  CHECK(Hq >= 1 && Hq % P == 0 && Hkv >= 1 && Hkv % P == 0, ULY_ERR_INVALID_ARG,
        "%s: Hq=%d and Hkv=%d must be positive multiples of P=%d", fn, Hq, Hkv, P);
  CHECK(Hq <= 4096 && Hkv <= 4096, ULY_ERR_INVALID_ARG, "%s: Hq=%d, Hkv=%d too large", fn, Hq, Hkv);
  CHECK(group >= 0 && group < P, ULY_ERR_INVALID_ARG, "%s: group=%d must be in [0, P=%d)", fn, group, P);
  uly::AttnDesc d;
  uly_status s = check_attn(fn, int64_t(P) * T, Hq / P, Hkv / P, D, dt, cu_seqlens, ndocs, softmax_scale, causal, &d);
  if (s != ULY_OK) return s;
  CHECK(dt == ULY_BF16, ULY_ERR_UNSUPPORTED, "%s: only bf16 inputs are read in place", fn);
  CHECK(T % 64 == 0, ULY_ERR_UNSUPPORTED, "%s: T=%lld must be a multiple of 64", fn, (long long)T);
  CHECK(q_shards != nullptr && k_shards != nullptr && v_shards != nullptr, ULY_ERR_INVALID_ARG,
        "%s: a shard array is NULL", fn);
  for (int j = 0; j < P; ++j)
    CHECK(q_shards[j] != nullptr && aligned16(q_shards[j]) && k_shards[j] != nullptr && aligned16(k_shards[j]) &&
              v_shards[j] != nullptr && aligned16(v_shards[j]),
          ULY_ERR_INVALID_ARG, "%s: shard %d of q, k or v is NULL or not 16-byte aligned", fn, j);
  CHECK(o != nullptr && aligned16(o) && lse != nullptr && aligned16(lse), ULY_ERR_INVALID_ARG,
        "%s: o or lse is NULL or not 16-byte aligned", fn);
  return from_hip(uly::launch_attn_fwd_from_shards(q_shards, k_shards, v_shards, P, T, Hq, Hkv, group, o, lse, d,
                                                   stream), fn);
}

uly_status attn_merge(const void* const* o_parts, const float* const* lse_parts, int nparts, int64_t N, int hq,
                      int D, uly_dtype dt, void* o, float* lse, hipStream_t stream) {
  CHECK(nparts >= 1 && nparts <= ULY_MAX_P, ULY_ERR_INVALID_ARG, "attn_merge: nparts=%d must be in [1, %d]", nparts,
        ULY_MAX_P);
  CHECK(N >= 1 && N <= (int64_t(1) << 30), ULY_ERR_INVALID_ARG, "attn_merge: N=%lld must be in [1, 2^30]",
        (long long)N);
  CHECK(hq >= 1 && hq <= 1024, ULY_ERR_INVALID_ARG, "attn_merge: hq=%d must be in [1, 1024]", hq);
  CHECK(D == 64 || D == 128, ULY_ERR_INVALID_ARG, "attn_merge: D=%d must be 64 or 128", D);
  CHECK(valid_dtype(dt), ULY_ERR_INVALID_ARG, "attn_merge: unknown dtype %d", (int)dt);
  CHECK(N * hq * D / 8 < (int64_t(1) << 31), ULY_ERR_UNSUPPORTED,
        "attn_merge: N * hq * D = %lld elements exceeds 2^34", (long long)(N * hq * D));
  CHECK(o_parts != nullptr && lse_parts != nullptr, ULY_ERR_INVALID_ARG, "attn_merge: o_parts or lse_parts is NULL");
  CHECK(o != nullptr && aligned16(o), ULY_ERR_INVALID_ARG, "attn_merge: o is NULL or not 16-byte aligned");
  CHECK(lse != nullptr && aligned16(lse), ULY_ERR_INVALID_ARG, "attn_merge: lse is NULL or not 16-byte aligned");
  for (int c = 0; c < nparts; ++c) {
    CHECK(o_parts[c] != nullptr && aligned16(o_parts[c]), ULY_ERR_INVALID_ARG,
          "attn_merge: o_parts[%d] is NULL or not 16-byte aligned", c);
    CHECK(lse_parts[c] != nullptr && aligned16(lse_parts[c]), ULY_ERR_INVALID_ARG,
          "attn_merge: lse_parts[%d] is NULL or not 16-byte aligned", c);
    CHECK(o_parts[c] != o && lse_parts[c] != lse, ULY_ERR_INVALID_ARG,
          "attn_merge: part %d aliases an output", c);
  }
  return from_hip(uly::launch_attn_merge(o_parts, lse_parts, nparts, N, hq, D, dt, o, lse, stream), "attn_merge");
}

uly_status attn_bwd_workspace_size(int64_t N, int hq, int hk, int D, uly_dtype dt, size_t* bytes) {
  uly::AttnDesc d;
  uly_status s = check_attn("attn_bwd_workspace_size", N, hq, hk, D, dt, nullptr, 1, 1.0f, 1, &d);
  if (s != ULY_OK) return s;
  CHECK(bytes != nullptr, ULY_ERR_INVALID_ARG, "attn_bwd_workspace_size: bytes is NULL");
  *bytes = uly::bwd_workspace_bytes(d);
  return ULY_OK;
}

}  // extern "C"

namespace {

uly_status bwd_common(const char* fn, int accumulate, const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, int64_t N, int hq, int hk,
                      int D, uly_dtype dt, const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, uly_dtype grad_dt) {
  uly::AttnDesc d;
  uly_status s = check_attn(fn, N, hq, hk, D, dt, cu_seqlens, ndocs, softmax_scale, causal, &d);
  if (s != ULY_OK) return s;
  CHECK(valid_dtype(grad_dt), ULY_ERR_INVALID_ARG, "%s: unknown grad_dt %d", fn, (int)grad_dt);
  CHECK(grad_dt == dt || grad_dt == ULY_F32, ULY_ERR_UNSUPPORTED,
        "%s: grad_dt must equal dt or be ULY_F32", fn);
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  const char* names[] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"};
  for (int i = 0; i < 9; ++i)
    CHECK(ptrs[i] != nullptr && aligned16(ptrs[i]), ULY_ERR_INVALID_ARG,
          "%s: %s is NULL or not 16-byte aligned", fn, names[i]);
  const size_t need = uly::bwd_workspace_bytes(d);
  CHECK(workspace_bytes >= need, ULY_ERR_INVALID_ARG, "%s: workspace_bytes=%zu < required %zu", fn,
        workspace_bytes, need);
  CHECK(need == 0 || (workspace != nullptr && aligned16(workspace)), ULY_ERR_INVALID_ARG,
        "%s: workspace is NULL or not 16-byte aligned", fn);
  d.accumulate = accumulate;
  return from_hip(uly::launch_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, d, grad_dt, stream), fn);
}

}  // namespace

extern "C" {

uly_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int64_t N, int hq, int hk, int D,
                    uly_dtype dt, const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_common("attn_bwd", 0, q, k, v, o, dout, lse, dq, dk, dv, N, hq, hk, D, dt, cu_seqlens, ndocs,
                    softmax_scale, causal, workspace, workspace_bytes, stream, dt);
}

uly_status attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int64_t N, int hq, int hk, int D,
                       uly_dtype dt, const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                       void* workspace, size_t workspace_bytes, hipStream_t stream, uly_dtype grad_dt) {
  return bwd_common("attn_bwd_ex", 0, q, k, v, o, dout, lse, dq, dk, dv, N, hq, hk, D, dt, cu_seqlens, ndocs,
                    softmax_scale, causal, workspace, workspace_bytes, stream, grad_dt);
}

uly_status attn_bwd_accumulate(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, int64_t N, int hq, int hk, int D,
                               uly_dtype dt, const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_common("attn_bwd_accumulate", 1, q, k, v, o, dout, lse, dq, dk, dv, N, hq, hk, D, dt, cu_seqlens,
                    ndocs, softmax_scale, causal, workspace, workspace_bytes, stream, ULY_F32);
}

uly_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, int64_t N, int hq, int hk, int D,
                            uly_dtype dt, const int32_t* cu_seqlens, int ndocs, float softmax_scale, int causal,
                            hipStream_t stream) {
  const char* fn = "attn_bwd_noalloc";
  uly::AttnDesc d;
  uly_status s = check_attn(fn, N, hq, hk, D, dt, cu_seqlens, ndocs, softmax_scale, causal, &d);
  if (s != ULY_OK) return s;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  const char* names[] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"};
  for (int i = 0; i < 9; ++i)
    CHECK(ptrs[i] != nullptr && aligned16(ptrs[i]), ULY_ERR_INVALID_ARG,
          "%s: %s is NULL or not 16-byte aligned", fn, names[i]);
  uly::AttnDesc one = d;
  one.splits = 1;
  const size_t need = uly::bwd_workspace_bytes(one);
  CHECK(need <= uly::kNoAllocScratchBytes, ULY_ERR_UNSUPPORTED,
        "%s: these sizes need %zu bytes of workspace, more than the %zu bytes of the static buffer", fn, need,
        uly::kNoAllocScratchBytes);
  size_t need2 = 0;
  const hipError_t e = uly::launch_attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, d, stream, &need2);
  if (e == hipErrorInvalidDevice)
    return fail(ULY_ERR_INVALID_ARG, "%s: the stream does not belong to the current device", fn);
  return from_hip(e, fn);
}

}  // extern "C"
