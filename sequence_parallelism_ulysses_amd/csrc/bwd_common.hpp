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
  const int32_t* cu;
  int ndocs;
  int N, hq, hk, G, Gw;
  int n_tiles;
  int splits;  // workgroups sharing one dK/dV key tile
  int causal;  // 1: key j visible to query i iff j <= i (and same document); 0: same document
  int accumulate;  // 1: add the gradients to dq, dk, dv (fp32 outputs only) instead of overwriting
  float scale, scale_log2;
};

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
template <int D, bool kF32Out>
hipError_t launch_dkdv_bf16(const BwdParams& p, dim3 grid, hipStream_t stream);

}  // namespace uly
