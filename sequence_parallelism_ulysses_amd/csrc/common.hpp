// Device helpers shared by the attention kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ulysses.h"

namespace uly {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32 output tile of a v_mfma_f32_32x32x* instruction, as held by lane l,
// accumulator slot r (checked on gfx950):
//   column = l % 32,  row = 8*(r/4) + 4*(l/32) + (r%4).
// Operand A (rows x k) is read by lane l as row l%32; operand B (k x cols) as
// column l%32; the k values a lane supplies are paired between A and B by
// lane half (l/32) and position within the lane.
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// fp16 variant of the same product. The backward of bf16 inputs runs its
// products on fp16 operands (11 significant bits against bf16's 8, same MFMA
// rate): inputs are copied to fp16 with a power-of-two scale per tensor, and
// the probabilities and dS are rounded to fp16 instead of bf16. The operands
// travel in the same 16-bit fragment type the LDS readers return.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16_t mfma_f16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// Combine a per-lane value with the same lane of the other half-wave
// (lane l and lane l^32): v_permlane32_swap hands each lane both values.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform value (lets the compiler keep it in an SGPR and branch on it).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Lazy rescaling of the online softmax: the running max is only raised (and
// the accumulators rescaled) when a new score exceeds it by more than 2^8, so
// unnormalised probabilities stay below 256 and most tiles skip the rescale.
constexpr float kRescaleLog2 = 8.f;

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> two bf16 in one 32-bit word (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> two fp16 (round to nearest even) in one 32-bit word
// (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}
// Eight fp32 values as an fp16 MFMA fragment (see mfma_f16).
__device__ __forceinline__ bf16x8_t make_frag_f16(const float* v) {
  u32x4_t w;
  w[0] = pack_f16x2(v[0], v[1]);
  w[1] = pack_f16x2(v[2], v[3]);
  w[2] = pack_f16x2(v[4], v[5]);
  w[3] = pack_f16x2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8_t, w);
}

// An offset of cu_seqlens clamped to [0, N]: malformed offsets (a documented
// precondition, not checked on the device) then only give wrong results,
// never index ranges outside the tensors.
__device__ __forceinline__ int cu_clamped(const int32_t* __restrict__ cu, int i, int N) {
  return min(max(int(cu[i]), 0), N);
}

// Document containing token t: offsets cu[0..ndocs] are non-decreasing from
// 0 to N, and t < N. Returns its [start, end), both within [0, N].
// cu == nullptr: one document.
struct DocSpan {
  int start, end;
};
__device__ __forceinline__ DocSpan doc_of(const int32_t* __restrict__ cu, int ndocs, int N, int t) {
  if (cu == nullptr) return {0, N};
  int lo = 0, hi = ndocs;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return {cu_clamped(cu, lo, N), cu_clamped(cu, hi, N)};
}

// Launch order by causal work with packed documents. Query tile q covers
// rows [q*R, (q+1)*R); under the causal mask its work grows with its
// position k = q - floor(cu_d / R) counted from the first tile of the
// document d that holds its first row. Tiles whose first row lies in
// document d have the keys a_d .. e_d, one tile each, with
//   a_d = ceil(cu_d / R) - floor(cu_d / R),  e_d = ceil(cu_{d+1} / R) - 1 - floor(cu_d / R),
// and these ranges cover all ceil(N / R) tiles once. Returns the tile of rank
// b (0-based) in the order (key descending, document descending): the key by
// a binary search on C(k) = number of tiles with key >= k, a sum over the
// documents with one lane per document, then the document by its rank among
// those holding that key. Every lane returns the same tile. Requires
// 1 <= ndocs <= 64 and valid cu_seqlens; without documents the order is
// simply q = n_tiles - 1 - b.
// The core takes this lane's document span [c0, c1) (has_doc false: no
// document on this lane); the spans must tile [0, n_tiles*R) or [0, N).
__device__ __forceinline__ int tile_by_work_rank_spans(bool has_doc, int c0, int c1, int R, int n_tiles, int b) {
  const int lane = threadIdx.x & 63;
  int a = 1, e = 0, base = 0;  // lanes without a document hold an empty range
  if (has_doc) {
    base = c0 / R;
    a = (c0 + R - 1) / R - base;
    e = (c1 + R - 1) / R - 1 - base;
  }
  auto count_ge = [&](int k) {
    const int lo = a > k ? a : k;
    int c = e >= lo ? e - lo + 1 : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m);
    return c;
  };
  // largest key k with C(k) > b: C(0) = n_tiles > b and C(n_tiles) = 0
  int lo = 0, hi = n_tiles;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (count_ge(mid) > b) lo = mid; else hi = mid;
  }
  const int j = b - count_ge(lo + 1);  // rank among the documents holding key lo
  const bool has = has_doc && a <= lo && lo <= e;
  const uint64_t mask = __ballot(has);
  const int above = __popcll((mask >> lane) >> 1);  // documents after this lane's holding key lo
  const uint64_t pick = __ballot(has && above == j);
  const int d = pick ? __ffsll(static_cast<unsigned long long>(pick)) - 1 : 0;
  const int q = __shfl(base, d) + lo;
  return q < 0 ? 0 : (q >= n_tiles ? n_tiles - 1 : q);
}

__device__ __forceinline__ int tile_by_work_rank(const int32_t* __restrict__ cu, int ndocs, int N, int R,
                                                 int n_tiles, int b) {
  const int lane = threadIdx.x & 63;
  const bool has_doc = lane < ndocs;
  return tile_by_work_rank_spans(has_doc, has_doc ? cu_clamped(cu, lane, N) : 0,
                                 has_doc ? cu_clamped(cu, lane + 1, N) : 0, R, n_tiles, b);
}

// The same order for key blocks of R keys under the causal mask, whose work
// grows with their distance from the end of the document holding their last
// key: rank the blocks of the mirrored sequence (token p -> n_tiles*R - 1 - p,
// where the R-aligned padding past N becomes a leading empty document) and
// map back. Requires ndocs + 1 <= 64.
__device__ __forceinline__ int key_block_by_work_rank(const int32_t* __restrict__ cu, int ndocs, int N, int R,
                                                      int n_tiles, int b) {
  const int lane = threadIdx.x & 63;
  const int npad = n_tiles * R;
  // mirrored document l: l = 0 the padding [0, npad - N), l >= 1 the original
  // document ndocs - l
  const bool has_doc = lane <= ndocs;
  int c0 = 0, c1 = 0;
  if (has_doc) {
    c0 = lane == 0 ? 0 : npad - cu_clamped(cu, ndocs - lane + 1, N);
    c1 = lane == 0 ? npad - N : npad - cu_clamped(cu, ndocs - lane, N);
  }
  return n_tiles - 1 - tile_by_work_rank_spans(has_doc, c0, c1, R, n_tiles, b);
}

// Element traits: bf16 uses v_mfma_f32_32x32x16_bf16 (8 k-values per lane),
// fp32 uses v_mfma_f32_32x32x2f32 (1 k-value per lane).
struct TrBF16 {
  using frag_t = bf16x8_t;
  static constexpr int kElem = 2;
  static constexpr int kStep = 16;  // k per instruction
  static constexpr int kEpl = 8;    // k values per lane
  static constexpr uly_dtype kDtype = ULY_BF16;
};
struct TrF32 {
  using frag_t = float;
  static constexpr int kElem = 4;
  static constexpr int kStep = 2;
  static constexpr int kEpl = 1;
  static constexpr uly_dtype kDtype = ULY_F32;
};

// Load one operand fragment (kEpl contiguous elements) from a byte address.
template <class Tr>
__device__ __forceinline__ typename Tr::frag_t load_frag(const void* p) {
  return *reinterpret_cast<const typename Tr::frag_t*>(p);
}

// Build a fragment from kEpl fp32 values (rounded to bf16 for TrBF16).
template <class Tr>
__device__ __forceinline__ typename Tr::frag_t make_frag(const float* v);
template <>
__device__ __forceinline__ bf16x8_t make_frag<TrBF16>(const float* v) {
  u32x4_t w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  w[2] = pack_bf16x2(v[4], v[5]);
  w[3] = pack_bf16x2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8_t, w);
}
template <>
__device__ __forceinline__ float make_frag<TrF32>(const float* v) { return v[0]; }

}  // namespace uly
