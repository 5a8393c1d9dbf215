// Merge of partial attention results over disjoint key chunks.
//
// The pages compare Ulysses with Ring Attention, which passes key/value
// chunks around a ring of GPUs ("Snowflake's Ulysses trick ...", third
// paragraph); each step yields, for the local queries, the attention output
// and log-sum-exp over one chunk of keys. Softmax over a union of disjoint
// key sets combines exactly from those per-chunk results:
//   lse   = log sum_c exp(lse_c)
//   o     = sum_c exp(lse_c - lse) o_c
// computed here in fp32 (max-shifted), one pass over the parts.
//
// HBM-bound: each thread owns 8 consecutive elements (16 bytes of bf16, 32 of
// fp32) of one (row, head) vector and streams the same slice of every part;
// the D/8 threads of a vector share its lse values through the cache, and
// the first of them writes the merged lse.
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace uly {
namespace {

constexpr int kThreads = 256;

struct MergeArgs {
  const char* o_part[ULY_MAX_P];
  const float* lse_part[ULY_MAX_P];
  char* o;
  float* lse;
  int nparts;
  int N, hq, D;
  uint64_t n_threads;  // N * hq * D / 8
};

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  const uint64_t t = uint64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= a.n_threads) return;
  const int per_vec = a.D / 8;
  const uint64_t vec = t / per_vec;              // (row, head) in [N][hq] order
  const int slice = int(t - vec * per_vec);       // which 8 elements of D
  const int row = int(vec / a.hq), head = int(vec - uint64_t(row) * a.hq);
  const uint64_t lse_at = uint64_t(head) * a.N + row;
  constexpr int E = kBf16 ? 2 : 4;
  const uint64_t byte_at = (vec * a.D + uint64_t(slice) * 8) * E;

  float m = -INFINITY;
  for (int c = 0; c < a.nparts; ++c) m = fmaxf(m, a.lse_part[c][lse_at]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int c = 0; c < a.nparts; ++c) {
      const float w = __expf(a.lse_part[c][lse_at] - m);  // 0 for a part with lse -inf
      wsum += w;
      const char* src = a.o_part[c] + byte_at;
      if constexpr (kBf16) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += w * bf16_bits_to_f32(v[i] & 0xffffu);
          acc[2 * i + 1] += w * bf16_bits_to_f32(v[i] >> 16);
        }
      } else {
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(src);
        const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(src + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += w * __uint_as_float(v0[i]);
          acc[4 + i] += w * __uint_as_float(v1[i]);
        }
      }
    }
  }
  // every part empty (all lse -inf): o = 0, lse = -inf
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  char* dst = a.o + byte_at;
  if constexpr (kBf16) {
    *reinterpret_cast<u32x4_t*>(dst) =
        u32x4_t{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  } else {
    *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{__float_as_uint(acc[0] * inv), __float_as_uint(acc[1] * inv),
                                               __float_as_uint(acc[2] * inv), __float_as_uint(acc[3] * inv)};
    *reinterpret_cast<u32x4_t*>(dst + 16) = u32x4_t{__float_as_uint(acc[4] * inv), __float_as_uint(acc[5] * inv),
                                                    __float_as_uint(acc[6] * inv), __float_as_uint(acc[7] * inv)};
  }
  if (slice == 0) a.lse[lse_at] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(const void* const* o_parts, const float* const* lse_parts, int nparts, int64_t N,
                             int hq, int D, uly_dtype dt, void* o, float* lse, hipStream_t stream) {
  MergeArgs a{};
  for (int c = 0; c < nparts; ++c) {
    a.o_part[c] = static_cast<const char*>(o_parts[c]);
    a.lse_part[c] = lse_parts[c];
  }
  a.o = static_cast<char*>(o);
  a.lse = lse;
  a.nparts = nparts;
  a.N = static_cast<int>(N);
  a.hq = hq;
  a.D = D;
  a.n_threads = static_cast<uint64_t>(N) * hq * D / 8;
  const dim3 grid(static_cast<unsigned>((a.n_threads + kThreads - 1) / kThreads));
  if (dt == ULY_BF16)
    merge_kernel<true><<<grid, kThreads, 0, stream>>>(a);
  else
    merge_kernel<false><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace uly
