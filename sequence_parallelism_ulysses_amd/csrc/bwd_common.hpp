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
  float scale, scale_log2;
};

// Store 4 consecutive gradient values as fp32 (16 bytes) or bf16 (8 bytes,
// rounded to nearest even).
template <bool kF32>
__device__ __forceinline__ void store4(char* dst, const float (&x)[4]) {
  if constexpr (kF32) {
    *reinterpret_cast<u32x4_t*>(dst) =
        u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
  } else {
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  }
}

// bf16 dK/dV kernel (its own translation unit, compiled with its own
// scheduling flags); launches on `stream` and returns the launch status.
template <int D, bool kF32Out>
hipError_t launch_dkdv_bf16(const BwdParams& p, dim3 grid, hipStream_t stream);

}  // namespace uly
