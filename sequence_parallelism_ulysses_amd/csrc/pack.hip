// Sequence <-> head redistribution for one head group (the local halves of
// the two all-to-alls in "Snowflake's Ulysses trick trains transformers on
// million-token contexts across GPUs", second paragraph).
//
// Both directions move the same bytes: for every global token n = j*T + t the
// head group's hh*D elements form one contiguous segment in shard j (at byte
// t*row_bytes + head_offset) and one contiguous segment in the packed buffer
// (at byte n*seg_bytes). Segments are a multiple of 16 bytes, so the kernel
// copies 16-byte chunks: in the packed buffer, chunk i of shard j's block sits
// at byte (j*T*seg_bytes + 16*i), so that side is one dense stream; the shard
// side is a run of seg_bytes-long contiguous pieces.
//
// HBM-bound (no arithmetic): each thread keeps kItems 16-byte loads in flight
// before it stores, consecutive lanes touch consecutive chunks (full 64-byte
// lines per 4 lanes), loads and stores are non-temporal, and one grid row per
// shard keeps the shard pointer uniform across the workgroup.
#include "internal.hpp"

namespace uly {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;  // 16-byte chunks per thread

struct PermuteArgs {
  char* shard[ULY_MAX_P];
  char* packed;
  uint32_t T;               // tokens per shard
  uint32_t chunks_per_row;  // seg_bytes / 16
  uint64_t row_bytes;
  uint64_t seg_bytes;
  uint64_t head_offset;
};

typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));  // one 16-byte chunk

template <bool kPack>
__global__ __launch_bounds__(kThreads) void permute_kernel(PermuteArgs a) {
  const uint32_t j = blockIdx.y;
  const uint32_t n_chunks = a.T * a.chunks_per_row;  // < 2^31, checked on the host
  char* shard = a.shard[j];
  char* packed = a.packed + (uint64_t)j * a.T * a.seg_bytes;
  const uint32_t first = blockIdx.x * (kThreads * kItems);
  const uint32_t base = first + threadIdx.x;

  auto shard_off = [&](uint32_t i) {
    const uint32_t t = i / a.chunks_per_row;
    const uint32_t c = i - t * a.chunks_per_row;
    return (uint64_t)t * a.row_bytes + a.head_offset + 16ull * c;
  };
  // Every byte is touched once: non-temporal loads and stores keep the
  // stream from displacing cache lines that other work still needs (and on
  // MI355X move about 40 % more bytes per second than plain ones here).
  auto load = [&](uint32_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const chunk_t*>(kPack ? shard + shard_off(i) : packed + 16ull * i));
  };
  auto store = [&](uint32_t i, chunk_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<chunk_t*>(kPack ? packed + 16ull * i : shard + shard_off(i)));
  };

  if (first + kThreads * kItems <= n_chunks) {
    // whole block in range: all kItems loads in flight before the first store
    // (named registers; a guarded array here ends up staged through memory)
    static_assert(kItems == 8, "the fast path names its eight chunks");
    const chunk_t v0 = load(base), v1 = load(base + kThreads), v2 = load(base + 2 * kThreads),
                  v3 = load(base + 3 * kThreads), v4 = load(base + 4 * kThreads), v5 = load(base + 5 * kThreads),
                  v6 = load(base + 6 * kThreads), v7 = load(base + 7 * kThreads);
    store(base, v0);
    store(base + kThreads, v1);
    store(base + 2 * kThreads, v2);
    store(base + 3 * kThreads, v3);
    store(base + 4 * kThreads, v4);
    store(base + 5 * kThreads, v5);
    store(base + 6 * kThreads, v6);
    store(base + 7 * kThreads, v7);
  } else {
    for (uint32_t i = base; i < n_chunks; i += kThreads) store(i, load(i));
  }
}

PermuteArgs make_args(const PermuteDesc& d) {
  PermuteArgs a{};
  a.T = static_cast<uint32_t>(d.T);
  a.chunks_per_row = static_cast<uint32_t>(d.seg_bytes / 16);
  a.row_bytes = d.row_bytes;
  a.seg_bytes = d.seg_bytes;
  a.head_offset = d.head_offset;
  return a;
}

dim3 grid_for(const PermuteDesc& d) {
  const uint64_t n_chunks = static_cast<uint64_t>(d.T) * (d.seg_bytes / 16);
  const uint64_t per_block = kThreads * kItems;
  return dim3(static_cast<unsigned>((n_chunks + per_block - 1) / per_block),
              static_cast<unsigned>(d.P), 1);
}

}  // namespace

hipError_t launch_pack(const void* const* shards, void* out, const PermuteDesc& d,
                       hipStream_t stream) {
  PermuteArgs a = make_args(d);
  for (int j = 0; j < d.P; ++j) a.shard[j] = const_cast<char*>(static_cast<const char*>(shards[j]));
  a.packed = static_cast<char*>(out);
  permute_kernel<true><<<grid_for(d), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_unpack(const void* in, void* const* shards, const PermuteDesc& d,
                         hipStream_t stream) {
  PermuteArgs a = make_args(d);
  for (int j = 0; j < d.P; ++j) a.shard[j] = static_cast<char*>(shards[j]);
  a.packed = const_cast<char*>(static_cast<const char*>(in));
  permute_kernel<false><<<grid_for(d), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace uly
