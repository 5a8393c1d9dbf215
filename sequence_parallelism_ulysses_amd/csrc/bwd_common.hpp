// Shared by the attention backward translation units.
#pragma once

#include "common.hpp"
#include "internal.hpp"
#include "lds_tile.hpp"

namespace uly {

constexpr int BT = 64;  // rows of a staged Q/dO tile (dK/dV) or K/V tile (dQ)

struct BwdParams {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;
  const float* lse;
  char* dq;
  char* dk;
  char* dv;
  float* delta;
  float* lse2;     // lse * log2(e), [hq][N]
  float* part_dk;  // [splits][N][hk][D] fp32, when splits > 1
  float* part_dv;
  // bf16 inputs: fp16 copies of q, dout ([N][hq][D]) and k, v ([N][hk][D]),
  // each scaled by a power of two, and the largest |value| of each input
  // tensor (bf16 bits: q, k, v, dout) that the scales derive from
  char* q16;
  char* do16;
  char* k16;
  char* v16;
  uint32_t* absmax;
  const int32_t* cu;
  int ndocs;
  int N, hq, hk, G, Gw;
  int n_tiles;
  int splits;  // workgroups sharing one dK/dV key tile
  int causal;  // 1: key j visible to query i iff j <= i (and same document); 0: same document
  int accumulate;  // 1: add the gradients to dq, dk, dv (fp32 outputs only) instead of overwriting
  float scale, scale_log2;
};

// Power-of-two scales of the fp16 operands of the bf16-input backward.
// Tensor x (q, k, v, dout) with max |x| < 2^kx is stored as x * 2^sx with
// sx <= 15 - kx, so its fp16 copy stays below 2^15 (fp16's largest finite
// value is 65504) and keeps bf16's 8 significant bits exactly down to at
// least 2^-21 of its largest value. The products then carry 2^(sq+sk) (S) and
// 2^(sdo+sv) (dP). With P <= 1, |dP_ij| <= |dO_i| |v_j| and |delta_i| <=
// |dO_i| |O_i| <= |dO_i| max_j |v_j| (row 2-norms; O is a convex combination
// of the v rows), |dS| <= 2.01 max|dO| max|v| < 2^(ndo+nv+2) for row norms
// below 2^ndo and 2^nv, so dS is stored as dS * 2^eds with eds <= 13 - ndo -
// nv, and P as P * 2^15. Each exponent is rounded down to a multiple of 8: for
// data of ordinary range (unit-scale inputs, or inputs a few times larger)
// the scales then do not move when some values change, so that results
// depend on other rows' data only where the mathematics says so. Every scale
// is exact, and each output is scaled back once in its epilogue.
struct BwdScales {
  float c_s;     // scale*log2(e)*2^-(sq+sk): S in exp2 units
  float kd;      // 2^(eds-15-sdo-sv): dP in the units of delta * 2^(eds-15)
  float mul_dq;  // scale * 2^-(eds+sk)
  float mul_dk;  // scale * 2^-(eds+sq)
  float mul_dv;  // 2^-(15+sdo)
};

// Slots of the maxima in the workspace (uint32 index, 256 bytes apart):
// max |x| as bf16 bits for q, k, v, dout, then the largest squared row norm
// (fp32 bits) of dout and v.
enum { kMaxQ = 0, kMaxK = 64, kMaxV = 128, kMaxDo = 192, kNormDo = 256, kNormV = 320, kMaxSlots = kBwdMaxima };

// Exponent bound of a bf16 |value| bit pattern: |x| < 2^k. Zero and
// subnormals give -126; inf/NaN give 0 (the results are not finite anyway).
__host__ __device__ __forceinline__ int exp_bound_bf16(uint32_t bits) {
  const int e = int((bits >> 7) & 0xff);
  if (e == 0xff) return 0;
  return e == 0 ? -126 : e - 126;
}
// Exponent bound of a norm from its square (fp32 bits): |x| < 2^k.
__host__ __device__ __forceinline__ int exp_bound_norm2(uint32_t bits) {
  const int e = int((bits >> 23) & 0xff);
  if (e == 0xff) return 0;
  const int e2 = e == 0 ? -126 : e - 126;  // norm^2 < 2^e2
  return (e2 + 1) >> 1;                     // ceil(e2 / 2)
}
// The largest multiple of 8 not above x, within the fp32 exponent range.
__host__ __device__ __forceinline__ int quant_exp(int x) {
  const int q = x >= 0 ? x / 8 * 8 : -((-x + 7) / 8 * 8);
  return q < -120 ? -120 : (q > 120 ? 120 : q);
}
__host__ __device__ __forceinline__ int fp16_scale_exp(uint32_t max_bits) {
  return quant_exp(15 - exp_bound_bf16(max_bits));
}
__host__ __device__ __forceinline__ int ds_scale_exp(uint32_t norm2_do_bits, uint32_t norm2_v_bits) {
  return quant_exp(13 - exp_bound_norm2(norm2_do_bits) - exp_bound_norm2(norm2_v_bits));
}

__device__ __forceinline__ BwdScales bwd_scales(const uint32_t* absmax, float scale) {
  const int sq = fp16_scale_exp(absmax[kMaxQ]), sk = fp16_scale_exp(absmax[kMaxK]);
  const int sv = fp16_scale_exp(absmax[kMaxV]), sdo = fp16_scale_exp(absmax[kMaxDo]);
  const int eds = ds_scale_exp(absmax[kNormDo], absmax[kNormV]);
  BwdScales b;
  b.c_s = ldexpf(scale * kLog2e, -(sq + sk));
  b.kd = ldexpf(1.f, eds - 15 - sdo - sv);
  b.mul_dq = ldexpf(scale, -(eds + sk));
  b.mul_dk = ldexpf(scale, -(eds + sq));
  b.mul_dv = ldexpf(1.f, -(15 + sdo));
  return b;
}

// Visibility bounds of a query-stationary wave (32 rows from qbase, last
// valid row wq_last): row i sees keys [doc start, hi(i)], hi(i) = i when
// causal, else the last token of i's document.
struct QueryBounds {
  int my_ds, my_hi;            // this lane's row
  int w_ds_first, w_ds_last;   // document starts of the wave's first and last rows
  int w_hi_first, w_hi_last;   // hi of the wave's first and last rows
  __device__ __forceinline__ QueryBounds(const BwdParams& p, int my_q, int qbase, int wq_last, bool active) {
    const DocSpan mine = doc_of(p.cu, p.ndocs, p.N, min(my_q, p.N - 1));
    const DocSpan first = doc_of(p.cu, p.ndocs, p.N, min(qbase, p.N - 1));
    const DocSpan last = doc_of(p.cu, p.ndocs, p.N, wq_last);
    my_ds = mine.start;
    my_hi = p.causal ? my_q : mine.end - 1;
    // wave-uniform (the inputs are), kept in scalar registers
    w_ds_first = uniform(active ? first.start : 0);
    w_ds_last = uniform(last.start);
    w_hi_first = uniform(p.causal ? qbase : first.end - 1);
    w_hi_last = uniform(p.causal ? wq_last : last.end - 1);
  }
};

// Visibility bounds of a key-stationary wave (32 keys from kw0): key j is
// seen by queries [lo(j), end of j's document), lo(j) = j when causal, else
// the first token of j's document.
struct KeyBounds {
  int my_lo, my_de;            // this lane's key
  int w_lo_first, w_lo_last;   // lo of the wave's first and last keys
  int w_de_first, w_de_last;   // document ends of the wave's first and last keys
  __device__ __forceinline__ KeyBounds(const BwdParams& p, int key, int kw0) {
    const DocSpan mine = doc_of(p.cu, p.ndocs, p.N, min(key, p.N - 1));
    const DocSpan first = doc_of(p.cu, p.ndocs, p.N, min(kw0, p.N - 1));
    const DocSpan last = doc_of(p.cu, p.ndocs, p.N, min(kw0 + 31, p.N - 1));
    my_lo = p.causal ? key : mine.start;
    my_de = mine.end;
    // wave-uniform (the inputs are), kept in scalar registers
    w_lo_first = uniform(p.causal ? kw0 : first.start);
    w_lo_last = uniform(p.causal ? kw0 + 31 : last.start);
    w_de_first = uniform(first.end);
    w_de_last = uniform(last.end);
  }
};

// First query that can see any key of [k0, ...): k0 itself when causal,
// else the start of k0's document.
__device__ __forceinline__ int first_query(const BwdParams& p, int k0) {
  return p.causal ? k0 : doc_of(p.cu, p.ndocs, p.N, min(k0, p.N - 1)).start;
}

// Store 4 consecutive gradient values as fp32 (16 bytes) or bf16 (8 bytes,
// rounded to nearest even). With `add` (fp32 only) the values are added to
// what the destination holds.
template <bool kF32>
__device__ __forceinline__ void store4(char* dst, const float (&x)[4], bool add = false) {
  if constexpr (kF32) {
    float y[4] = {x[0], x[1], x[2], x[3]};
    if (add) {
      const f32x4_t old = *reinterpret_cast<const f32x4_t*>(dst);
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = old[j] + y[j];
    }
    *reinterpret_cast<u32x4_t*>(dst) =
        u32x4_t{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
  } else {
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  }
}

// bf16 dK/dV kernel (its own translation unit, compiled with its own
// scheduling flags); launches on `stream` and returns the launch status.
// Sets p.n_tiles to the kernel's key blocks and launches splits of each for
// the hk kv heads.
template <int D, bool kF32Out>
hipError_t launch_dkdv_bf16(BwdParams& p, int splits, int hk, hipStream_t stream);

}  // namespace uly
