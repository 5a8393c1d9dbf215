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
// lines per 4 lanes), loads and stores are non-temporal, and every workgroup
// stays within one shard, so the shard pointer is uniform across it.
//
// One launch can move up to three segments, each with its own shard
// tensors, token size, head offset and packed tensor: the Q, K and V heads of
// a fused QKV projection output (same shards), or separate Q, K and V
// tensors. The grid's x range is split into consecutive block ranges, one
// per segment, so every workgroup copies chunks of a single segment.
#include "internal.hpp"

namespace uly {
namespace {

constexpr int kThreads = 256;
// 16-byte chunks per thread. Few chunks per thread and many small
// workgroups beat long per-thread runs here: measured on plain copies of
// 128 MiB to 1 GiB with the caches flushed, 4 chunks per thread reach 5.6 to
// 6.2 TB/s where 32 (named registers, all loads before all stores) reach 5.0
// to 5.3 TB/s.
constexpr int kItems = 4;
constexpr int kMaxSegments = 3;

struct Segment {
  char* shard[ULY_MAX_P];   // the P shard tensors this segment is read from / written to
  char* packed;             // [P*T][seg_bytes] packed tensor of this segment
  uint64_t row_bytes;       // bytes of one shard token (all its heads)
  uint64_t seg_bytes;       // bytes of one token's segment
  uint64_t head_offset;     // byte offset of the segment inside a shard token
  uint32_t chunks_per_row;  // seg_bytes / 16
  uint32_t block_begin;     // first blockIdx.x of this segment
  uint32_t blocks_per_shard;
};

struct PermuteArgs {
  Segment seg[kMaxSegments];
  uint32_t nseg;
  uint32_t T;               // tokens per shard
  uint32_t blocks;          // blocks of kThreads * kItems chunks over all segments and shards
};

// Workgroups of a launch: each loops over the blocks with a stride of the
// grid (8 per CU; on plain copies of 128 MiB to 1 GiB this is 1-5 % faster
// than one workgroup per block).
constexpr uint32_t kMaxGrid = 2048;

typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));  // one 16-byte chunk

template <bool kPack>
__global__ __launch_bounds__(kThreads) void permute_kernel(PermuteArgs a) {
  for (uint32_t vb = blockIdx.x; vb < a.blocks; vb += gridDim.x) {
    // the segment of this block (uniform index into the kernel arguments),
    // then its shard: blocks run segment by segment, each segment shard by
    // shard, as separate launches would
    const int s = int(a.nseg > 1 && vb >= a.seg[1].block_begin) + int(a.nseg > 2 && vb >= a.seg[2].block_begin);
    const Segment& sg = a.seg[s];
    const uint32_t local = vb - sg.block_begin;
    const uint32_t j = local / sg.blocks_per_shard;
    const uint32_t block_in_shard = local - j * sg.blocks_per_shard;
    const uint32_t cpr = sg.chunks_per_row;
    const uint64_t row_bytes = sg.row_bytes, head_offset = sg.head_offset;
    const uint32_t n_chunks = a.T * cpr;  // < 2^31, checked on the host
    char* shard = sg.shard[j];
    char* packed = sg.packed + (uint64_t)j * a.T * sg.seg_bytes;
    const uint32_t first = block_in_shard * (kThreads * kItems);
    const uint32_t base = first + threadIdx.x;

    auto shard_off = [&](uint32_t i) {
      const uint32_t t = i / cpr;
      const uint32_t c = i - t * cpr;
      return (uint64_t)t * row_bytes + head_offset + 16ull * c;
    };
    // Every byte is touched once: non-temporal loads and stores keep the
    // stream from displacing cache lines that other work still needs (and on
    // MI355X move about 40 % more bytes per second than plain ones here).
    auto load = [&](uint32_t i) {
      return __builtin_nontemporal_load(
          reinterpret_cast<const chunk_t*>(kPack ? shard + shard_off(i) : packed + 16ull * i));
    };
    auto store = [&](uint32_t i, chunk_t v) {
      __builtin_nontemporal_store(v, reinterpret_cast<chunk_t*>(kPack ? packed + 16ull * i : shard + shard_off(i)));
    };

    if (first + kThreads * kItems <= n_chunks) {
      // whole block in range: all kItems loads in flight before the first store
      chunk_t v[kItems];
#pragma unroll
      for (int k = 0; k < kItems; ++k) v[k] = load(base + k * kThreads);
#pragma unroll
      for (int k = 0; k < kItems; ++k) store(base + k * kThreads, v[k]);
    } else {
      // the last, partial block of a shard
      for (uint32_t i = base; i < n_chunks; i += kThreads) store(i, load(i));
    }
  }
}

uint32_t blocks_for(int64_t T, int64_t seg_bytes) {
  const uint64_t n_chunks = static_cast<uint64_t>(T) * static_cast<uint64_t>(seg_bytes / 16);
  const uint64_t per_block = kThreads * kItems;
  return static_cast<uint32_t>((n_chunks + per_block - 1) / per_block);
}

// Fill the launch arguments for the segments of `d`: segment s moves between
// the shards shard_ptrs[s][0..P) and the packed tensor packed[s]. Returns the
// grid: one range of blocks per segment, shard-major inside it.
dim3 make_args(const PermuteDesc& d, char* const* const* shard_ptrs, char* const* packed, PermuteArgs& a) {
  a = PermuteArgs{};
  a.T = static_cast<uint32_t>(d.T);
  a.nseg = static_cast<uint32_t>(d.nseg);
  uint32_t blocks = 0;
  for (int s = 0; s < d.nseg; ++s) {
    for (int j = 0; j < d.P; ++j) a.seg[s].shard[j] = shard_ptrs[s][j];
    a.seg[s].packed = packed[s];
    a.seg[s].row_bytes = static_cast<uint64_t>(d.row_bytes[s]);
    a.seg[s].seg_bytes = static_cast<uint64_t>(d.seg_bytes[s]);
    a.seg[s].head_offset = static_cast<uint64_t>(d.head_offset[s]);
    a.seg[s].chunks_per_row = static_cast<uint32_t>(d.seg_bytes[s] / 16);
    a.seg[s].block_begin = blocks;
    a.seg[s].blocks_per_shard = blocks_for(d.T, d.seg_bytes[s]);
    blocks += a.seg[s].blocks_per_shard * static_cast<uint32_t>(d.P);
  }
  a.blocks = blocks;
  return dim3(blocks < kMaxGrid ? blocks : kMaxGrid, 1, 1);
}

}  // namespace

hipError_t launch_pack(const void* const* const* shards, void* const* out, const PermuteDesc& d,
                       hipStream_t stream) {
  static_assert(kMaxSegments == ULY_PERMUTE_MAX_SEGMENTS, "segment count");
  PermuteArgs a;
  char* packed[kMaxSegments] = {};
  char* const* shard_ptrs[kMaxSegments] = {};
  for (int s = 0; s < d.nseg; ++s) {
    packed[s] = static_cast<char*>(out[s]);
    shard_ptrs[s] = reinterpret_cast<char* const*>(const_cast<void* const*>(shards[s]));
  }
  const dim3 grid = make_args(d, shard_ptrs, packed, a);
  permute_kernel<true><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_unpack(const void* const* in, void* const* const* shards, const PermuteDesc& d,
                         hipStream_t stream) {
  PermuteArgs a;
  char* packed[kMaxSegments] = {};
  char* const* shard_ptrs[kMaxSegments] = {};
  for (int s = 0; s < d.nseg; ++s) {
    packed[s] = const_cast<char*>(static_cast<const char*>(in[s]));
    shard_ptrs[s] = reinterpret_cast<char* const*>(shards[s]);
  }
  const dim3 grid = make_args(d, shard_ptrs, packed, a);
  permute_kernel<false><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace uly
