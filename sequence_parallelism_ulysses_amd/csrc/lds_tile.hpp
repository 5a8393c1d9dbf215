// LDS tiles for the bf16 attention kernels (gfx950).
//
// A tile holds 64 consecutive token rows of one head of a [N][H][D] bf16
// tensor, row-major in LDS (2*D bytes per row, no padding). The 16-byte chunk
// index inside a row is XOR-swizzled by a function of the row so that both
// ways the kernels read a tile are bank-conflict free:
//   - ds_read_b128 of an MFMA operand: 16 consecutive rows, same chunk;
//   - ds_read_b64_tr_b16 of a transposed operand: 4 consecutive rows x one
//     aligned 64-byte block per half-wave.
// Tiles are filled by buffer_load ... lds (16 bytes per lane, written to
// consecutive LDS addresses), so each lane fetches the global chunk that the
// swizzle places at its LDS slot; rows past the end of the tensor are outside
// the buffer resource's range and read as zero.
#pragma once

#include "common.hpp"

namespace uly {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

template <int D>
struct TileFmt {
  static constexpr int kRows = 64;
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  static constexpr int kBytes = kRows * kRowBytes;
  static_assert(D == 64 || D == 128, "head dim");

  __device__ static __forceinline__ int swz(int row) {
    if constexpr (D == 128) {
      // rows 0..15 -> a permutation of 0..15 whose bits 2-3 differ for any 4 consecutive rows
      return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
      // 128-byte rows alternate bank halves; rows of equal parity get distinct chunks
      const int x = row >> 1;
      return ((x & 1) << 2) | ((x >> 1) & 3);
    }
  }
  // byte offset of logical chunk `chunk` of `row`
  __device__ static __forceinline__ int off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }
};

// Buffer resource over `bytes` bytes from `base`: loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The same, with both arguments moved to scalar registers (they must be
// wave-uniform), as inline assembly operands require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  // readfirstlane works on int: widen through uint32_t, never sign-extend
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b)));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b >> 32)));
  const uint64_t ub = (uint64_t(hi) << 32) | lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ub), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Asynchronous global -> LDS copy of kBytes (4 or 16) per lane: lane l's data
// lands at lds_wave_base + kBytes * l. Written as inline assembly, so the
// compiler does not know about the copy: it neither orders later LDS reads
// after it nor waits for it anywhere. The caller must wait for completion
// (vmcnt) and synchronise (barrier) before anyone reads the destination, and
// the resource must come from make_rsrc_uniform. M0, which holds the LDS base
// of the copy, is restored afterwards.
template <int kBytes>
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rsrc, const lds_char* lds_wave_base,
                                           uint32_t voffset) {
  static_assert(kBytes == 4 || kBytes == 16, "copy width");
  const uint32_t m = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds_wave_base))));
  uint32_t saved;
  if constexpr (kBytes == 16)
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved) : "s"(m), "v"(voffset), "s"(rsrc) : "memory");
  else
    __asm__ volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved) : "s"(m), "v"(voffset), "s"(rsrc) : "memory");
}

// Issue the asynchronous copy of one tile: rows [0, ROWS) of a tensor whose
// row r, head slice starts at byte r*row_stride from the resource base
// (rows past the resource's range read as zero). NT threads (tid in [0, NT))
// each issue ROWS*D*2/16/NT loads of 16 bytes; returns nothing, completion is
// counted by vmcnt in issue order. The row layout is that of TileFmt<D>
// whatever the number of rows.
// kOpaque: issue through dma_to_lds (rsrc from make_rsrc_uniform).
template <int D, int NT, int ROWS = 64, bool kOpaque = false>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rsrc, uint32_t row_stride, lds_char* tile, int tid) {
  using F = TileFmt<D>;
  constexpr int kLoads = ROWS * F::kChunks / NT;
  static_assert(ROWS * F::kChunks % NT == 0 && kLoads > 0, "tile split");
  const int lane = tid & 63, wave_base = tid & ~63;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int slot = NT * i + tid;               // 16-byte slot in the tile, consecutive per lane
    const int row = slot / F::kChunks;
    const int chunk = (slot % F::kChunks) ^ F::swz(row);  // logical chunk stored at this slot
    lds_char* dst = tile + 16 * (NT * i + wave_base);     // wave-uniform base; lane adds 16*lane
    (void)lane;
    if constexpr (kOpaque)
      dma_to_lds<16>(rsrc, dst, row * row_stride + chunk * 16);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)dst, 16,
                                               row * row_stride + chunk * 16, 0, 0, 0);
  }
}

template <int D, int NT, int ROWS = 64>
constexpr int tile_loads() { return ROWS * (D / 8) / NT; }

// Wait until at most `n` vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; exp/lgkm counters
// left at their maximum, i.e. not waited on).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// MFMA operand fragment (8 bf16 k-values per lane) for a 32-row block of a
// row-major tile: lane (row = r0 + l%32, half h) reads k = k0 + 8h .. +7,
// which are contiguous columns -> one ds_read_b128.
template <int D>
__device__ __forceinline__ bf16x8_t frag_rows(const lds_char* tile, int row, int k0, int half) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
      tile + TileFmt<D>::off(row, (k0 >> 3) + half));
}

// Transposed MFMA operand (32x32x16 A operand over the tile's rows): lane
// (m = col0 + l%32, half h) needs tile[k][m] for the 8 tile rows
// k = k0 + {4h..4h+3, 8+4h..8+4h+3}, i.e. the same k order as a fragment
// built from a 32x32 accumulator (rows 8*(r/4) + 4h + r%4). Two
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i%4 of the 8-byte piece read by lane 4j + i/4 (j = 0..3), so lane 4j + q
// of group g points at row k0 + 4h + j (+8) and columns
// col0 + 16*(g%2) + 4q .. +3.
template <int D>
__device__ __forceinline__ bf16x8_t frag_cols_tr(const lds_char* tile, int k0, int col0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int j = i >> 2, q = i & 3, h = g >> 1;
  const int col = col0 + 16 * (g & 1) + 4 * q;  // multiple of 4 -> half of a 16-byte chunk
  const int r0 = k0 + 4 * h + j;
  const int b0 = TileFmt<D>::off(r0, col >> 3) + ((col & 4) << 1);
  const int b1 = TileFmt<D>::off(r0 + 8, col >> 3) + ((col & 4) << 1);
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + b0));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + b1));
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Per-lane byte offsets of the fragments a wave reads from a tile, computed
// once outside the main loop so each LDS read in it is (stage base + a
// precomputed offset + an immediate).
//
// Row fragments (frag_rows): rows rb*32 + l%32, k = 16*ks + 8h. The swizzle
// of row rb*32 + l%32 equals that of l%32, so the offset of (rb, ks) is
// rows_off[ks] + rb*32*2D.
template <int D>
struct RowFragOffsets {
  int off[D / 16];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) off[ks] = TileFmt<D>::off(l32, 2 * ks + half);
  }
};

// Transposed fragments (frag_cols_tr) over tile rows k0 = 16*st (+0 / +8)
// and output columns col0 = 32*db: the swizzle of those rows does not depend
// on st, so the offset of (st, part, db) is off[part][db] + st*16*2D.
template <int D>
struct TrFragOffsets {
  int off[2][D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int j = i >> 2, q = i & 3, h = g >> 1;
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int col = 32 * db + 16 * (g & 1) + 4 * q;
        const int row = 4 * h + j + 8 * part;
        off[part][db] = TileFmt<D>::off(row, col >> 3) + ((col & 4) << 1);
      }
  }
};

// An LDS byte address held in a VGPR that the optimiser cannot see through:
// offsets added to it afterwards can only become the instruction's immediate
// offset field (this keeps per-read address arithmetic out of the loops).
__device__ __forceinline__ const lds_char* lds_base(const lds_char* tile, int byte_off) {
  uint32_t a = uint32_t(reinterpret_cast<uintptr_t>(tile)) + uint32_t(byte_off);
  __asm__("" : "+v"(a));
  return reinterpret_cast<const lds_char*>(uintptr_t(a));
}

template <int D>
__device__ __forceinline__ bf16x8_t frag_rows_at(const lds_char* tile, int byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(tile + byte_off);
}

__device__ __forceinline__ bf16x8_t frag_tr_at(const lds_char* tile, int off0, int off1) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off0));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off1));
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Transposed fragment from two precomputed bases plus a shared immediate.
__device__ __forceinline__ bf16x8_t frag_tr2(const lds_char* b0, const lds_char* b1, int imm) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b0 + imm));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b1 + imm));
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace uly
