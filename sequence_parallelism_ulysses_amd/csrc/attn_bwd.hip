// Causal (or document-only masked) GQA / packed-document attention backward
// for one head group.
//
// Gradients of L = sum(dO * O) for O = softmax(scale * Q K^T + mask) V, with
// the probabilities recomputed from the forward's log-sum-exp (training runs
// the attention step forward and backward; "Ulysses Sequence Parallelism:
// Training with Million-Token Contexts"):
//   delta_i = dO_i . O_i
//   P_ij = exp(scale q_i.k_j - lse_i),   dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - delta_i)
//   dV_j = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j
//
// Three kernels, all deterministic (no atomics):
//   1. delta: one row dot product per (query, head), and lse * log2(e).
//   2. dK/dV, key-stationary: a workgroup owns a block of keys of one kv
//      head (fp32: 128, bf16: 192), walks the query tiles that can see them
//      for every q head of the group, and sums the GQA heads in its
//      accumulators:
//        S  = Q K^T, dP = dO V^T   (A operand: Q/dO rows from LDS)
//        dV^T += dO^T P, dK^T += Q^T dS   (A operand: transposed Q/dO tiles)
//      The S/dP accumulators hold one key column per lane, which is the
//      B-operand layout the second pair of products needs. fp32 (this file):
//      4 waves of 32 keys, each doing all four products, on 64-query tiles.
//      bf16 (attn_bwd_dkdv.hip): 12 waves on 32-query tiles, split into
//      producers (S, dP, P, dS) and consumers (dV or dK) that pass P and dS
//      through LDS. With splits > 1 several workgroups share a key block and
//      write fp32 partials that dkdv_reduce_kernel adds in split order.
//   3. dQ, query-stationary: like the forward, a wave owns 32 query rows and
//      walks the key tiles: S^T = K Q^T, dP^T = V dO^T, then
//      dQ^T += K^T dS^T from a transposed K operand.
//
// Tiles: fp32 tiles are staged through registers into padded LDS rows (the
// transposed operand stored a second time); bf16 tiles are copied global ->
// LDS by buffer loads into row-major, XOR-swizzled rows (lds_tile.hpp) and
// the transposed operands are read with ds_read_b64_tr_b16.
#include <algorithm>
#include <cmath>
#include <numeric>

#include "bwd_common.hpp"

namespace uly {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;


constexpr int kKeysPerWg = 32 * kWaves;

__device__ __forceinline__ u32x4_t ld16(const char* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// ----------------------------------------------------------------------------
// 1. delta_i = dO_i . O_i  (fp32), for every (query, head). Each lane reads
//    16 bytes of the row, so a row takes D*E/16 lanes (8..32).
// ----------------------------------------------------------------------------
template <class Tr, int D>
__global__ __launch_bounds__(kThreads) void delta_kernel(BwdParams p) {
  constexpr int E = Tr::kElem;
  constexpr int LPR = D * E / 16;  // lanes per row
  static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row split");
  const int64_t row = int64_t(blockIdx.x) * (kThreads / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  const int64_t rows = int64_t(p.N) * p.hq;
  float acc = 0.f;
  if (row < rows) {
    const int64_t off = row * D * E + sub * 16;  // row = q * hq + h
    const u32x4_t x = ld16(p.o + off), y = ld16(p.dout + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (E == 2) {
        acc = fmaf(bf16_bits_to_f32(x[j] & 0xffffu), bf16_bits_to_f32(y[j] & 0xffffu), acc);
        acc = fmaf(bf16_bits_to_f32(x[j] >> 16), bf16_bits_to_f32(y[j] >> 16), acc);
      } else {
        acc = fmaf(__uint_as_float(x[j]), __uint_as_float(y[j]), acc);
      }
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && sub == 0) {
    const int64_t q = row / p.hq, h = row % p.hq;
    p.delta[h * p.N + q] = acc;
    p.lse2[h * p.N + q] = p.lse[h * p.N + q] * kLog2e;
  }
}

// bf16 inputs: the same delta and lse * log2(e) - 15 (the backward's P
// carries 2^15), plus what the fp16 operand scales derive from (BwdScales):
// the largest |value| of q, k, v and dout and the largest row norms of dout
// and v. A grid-stride loop over rows, so that each workgroup ends with one
// atomic max per quantity.
__device__ __forceinline__ uint32_t absmax_bf16x8(u32x4_t x) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max(m, max(x[j] & 0x7fffu, (x[j] >> 16) & 0x7fffu));
  return m;
}
__device__ __forceinline__ float sumsq_bf16x8(u32x4_t x) {
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = bf16_bits_to_f32(x[j] & 0xffffu), hi = bf16_bits_to_f32(x[j] >> 16);
    a = fmaf(lo, lo, fmaf(hi, hi, a));
  }
  return a;
}

template <int D>
__global__ __launch_bounds__(kThreads) void prep_bf16_kernel(BwdParams p) {
  constexpr int LPR = D * 2 / 16;       // lanes per row (16 bytes each)
  constexpr int RPB = kThreads / LPR;   // rows per workgroup and step
  const int sub = threadIdx.x % LPR;
  const int64_t rows_q = int64_t(p.N) * p.hq, rows_k = int64_t(p.N) * p.hk;
  // maxima as bit patterns of non-negative values (ordered like the values)
  uint32_t m[6] = {0, 0, 0, 0, 0, 0};  // q, k, v, dout (bf16 bits), |dout row|^2, |v row|^2 (fp32 bits)
  for (int64_t row0 = int64_t(blockIdx.x) * RPB; row0 < rows_q; row0 += int64_t(gridDim.x) * RPB) {
    const int64_t row = row0 + threadIdx.x / LPR;
    float acc = 0.f, nd = 0.f, nv = 0.f;
    if (row < rows_q) {
      const int64_t off = row * D * 2 + sub * 16;  // row = token * hq + head (or token * hk + head)
      const u32x4_t x = ld16(p.o + off), y = ld16(p.dout + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(bf16_bits_to_f32(x[j] & 0xffffu), bf16_bits_to_f32(y[j] & 0xffffu), acc);
        acc = fmaf(bf16_bits_to_f32(x[j] >> 16), bf16_bits_to_f32(y[j] >> 16), acc);
      }
      m[3] = max(m[3], absmax_bf16x8(y));
      nd = sumsq_bf16x8(y);
      m[0] = max(m[0], absmax_bf16x8(ld16(p.q + off)));
      if (row < rows_k) {
        const u32x4_t vv = ld16(p.v + off);
        m[1] = max(m[1], absmax_bf16x8(ld16(p.k + off)));
        m[2] = max(m[2], absmax_bf16x8(vv));
        nv = sumsq_bf16x8(vv);
      }
    }
#pragma unroll
    for (int s = LPR / 2; s >= 1; s >>= 1) {
      acc += __shfl_xor(acc, s, LPR);
      nd += __shfl_xor(nd, s, LPR);
      nv += __shfl_xor(nv, s, LPR);
    }
    m[4] = max(m[4], __float_as_uint(nd));
    m[5] = max(m[5], __float_as_uint(nv));
    if (row < rows_q && sub == 0) {
      const int64_t q = row / p.hq, h = row % p.hq;
      p.delta[h * p.N + q] = acc;
      p.lse2[h * p.N + q] = p.lse[h * p.N + q] * kLog2e - 15.f;
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1)
#pragma unroll
    for (int i = 0; i < 6; ++i) m[i] = max(m[i], uint32_t(__shfl_xor(int(m[i]), s)));
  __shared__ uint32_t wmax[kWaves][6];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int i = 0; i < 6; ++i) wmax[w][i] = m[i];
  __syncthreads();
  if (threadIdx.x < 6) {
    uint32_t x = 0;
    for (int i = 0; i < kWaves; ++i) x = max(x, wmax[i][threadIdx.x]);
    atomicMax(p.absmax + 64 * threadIdx.x, x);
  }
}

// Zero the maxima before prep_bf16_kernel (a kernel rather than a memset,
// so that the call can be captured in a graph).
__global__ void absmax_init_kernel(uint32_t* absmax) {
  if (threadIdx.x < kMaxSlots / 64) absmax[64 * threadIdx.x] = 0u;
}

// fp16 copies of q, dout, k and v, each scaled by its power of two
// (BwdScales), and delta rescaled to delta * 2^(eds-15). Every conversion is
// exact except the rounding of values below 2^-21 of a tensor's largest.
template <int D>
__global__ __launch_bounds__(kThreads) void convert_bf16_kernel(BwdParams p) {
  const float fq = ldexpf(1.f, fp16_scale_exp(p.absmax[kMaxQ])), fk = ldexpf(1.f, fp16_scale_exp(p.absmax[kMaxK]));
  const float fv = ldexpf(1.f, fp16_scale_exp(p.absmax[kMaxV])), fdo = ldexpf(1.f, fp16_scale_exp(p.absmax[kMaxDo]));
  const float fdl = ldexpf(1.f, ds_scale_exp(p.absmax[kNormDo], p.absmax[kNormV]) - 15);
  const int64_t nq = int64_t(p.N) * p.hq * D / 8, nk = int64_t(p.N) * p.hk * D / 8;  // 16-byte chunks
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < 2 * (nq + nk); i += stride) {
    const char* src;
    char* dst;
    float f;
    int64_t j = i;
    if (j < nq) { src = p.q; dst = p.q16; f = fq; }
    else if ((j -= nq) < nq) { src = p.dout; dst = p.do16; f = fdo; }
    else if ((j -= nq) < nk) { src = p.k; dst = p.k16; f = fk; }
    else { j -= nk; src = p.v; dst = p.v16; f = fv; }
    const u32x4_t x = ld16(src + 16 * j);
    u32x4_t y;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      y[w] = pack_f16x2(bf16_bits_to_f32(x[w] & 0xffffu) * f, bf16_bits_to_f32(x[w] >> 16) * f);
    *reinterpret_cast<u32x4_t*>(dst + 16 * j) = y;
  }
  const int64_t nd = int64_t(p.N) * p.hq;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < nd; i += stride) p.delta[i] *= fdl;
}

// ----------------------------------------------------------------------------
// 2. dK / dV (key-stationary)
// ----------------------------------------------------------------------------
// fp32 (the bf16 kernels are further down and in attn_bwd_dkdv.hip)
template <class Tr, int D>
struct KvCfg {
  static_assert(Tr::kElem == 4, "fp32 kernel");
  static constexpr int E = Tr::kElem;
  static constexpr int KS = D / Tr::kStep;   // MFMA steps over D
  static constexpr int DB = D / 32;
  // query rows per tile: 32 for D = 128, whose K/V rows and dK/dV
  // accumulators already take 256 registers per lane (64 would spill)
  static constexpr int QT = D == 128 ? 32 : 64;
  static constexpr int QB = QT / 32;          // 32-row blocks per tile
  static constexpr int QS = QT / Tr::kStep;   // MFMA steps over the queries of a tile
  // tiles are row-major with a 16-byte pad per row; transposed operands are
  // read element by element from them
  static constexpr int F_STRIDE = D * 4 + 16;
  static constexpr int X_BYTES = QT * F_STRIDE;           // one tile
  static constexpr int STAGE = 2 * X_BYTES + 2 * QT * 4;  // Q, dO, lse2, delta
  static constexpr int F_CH = QT * D * 4 / 16 / kThreads;  // 16-byte chunks per thread
};

template <class Tr, int D>
struct QTile {
  using C = KvCfg<Tr, D>;
  static constexpr int NR = C::F_CH;
  u32x4_t xq[NR], xd[NR];
  float lse2, dlt;

  __device__ __forceinline__ void load(const BwdParams& p, int head, int qs, int tid) {
    const int64_t row_bytes = int64_t(p.hq) * D * C::E;
    const char* qb = p.q + int64_t(head) * D * C::E;
    const char* db = p.dout + int64_t(head) * D * C::E;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 4), col = c % (D / 4);
      const int q = qs + row;
      const bool ok = q < p.N;
      xq[i] = ok ? ld16(qb + q * row_bytes + col * 16) : u32x4_t{0, 0, 0, 0};
      xd[i] = ok ? ld16(db + q * row_bytes + col * 16) : u32x4_t{0, 0, 0, 0};
    }
    if (tid < C::QT) {
      const int q = qs + tid;
      lse2 = q < p.N ? p.lse[int64_t(head) * p.N + q] * kLog2e : 0.f;
      dlt = q < p.N ? p.delta[int64_t(head) * p.N + q] : 0.f;
    }
  }

  __device__ __forceinline__ void store(char* st, int tid) const {
    char* qr = st;
    char* dr = st + C::X_BYTES;
    float* fl = reinterpret_cast<float*>(st + 2 * C::X_BYTES);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 4), col = c % (D / 4);
      *reinterpret_cast<u32x4_t*>(qr + row * C::F_STRIDE + col * 16) = xq[i];
      *reinterpret_cast<u32x4_t*>(dr + row * C::F_STRIDE + col * 16) = xd[i];
    }
    if (tid < C::QT) {
      fl[tid] = lse2;
      fl[C::QT + tid] = dlt;
    }
  }
};

template <class Tr, int D, bool kF32Out>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdParams p) {
  using C = KvCfg<Tr, D>;
  using frag_t = typename Tr::frag_t;
  constexpr int E = C::E;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int kvh = blockIdx.y;
  const int split = int(blockIdx.x) % p.splits;
  const int kv0 = (int(blockIdx.x) / p.splits) * (32 * kWaves);  // first tiles carry the most causal work
  const int kw0 = kv0 + 32 * w;
  const bool active = kw0 < p.N;
  const int key = kw0 + l32;
  const KeyBounds kbd(p, key, kw0);
  const int my_lo = kbd.my_lo, my_de = kbd.my_de;
  const int w_de_first = kbd.w_de_first, w_de_last = kbd.w_de_last;

  // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T.
  frag_t kf[C::KS], vf[C::KS];
  {
    const int64_t off = (int64_t(key) * p.hk + kvh) * D * E + half * Tr::kEpl * E;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      kf[ks] = key < p.N ? load_frag<Tr>(p.k + off + ks * Tr::kStep * E) : frag_t{};
      vf[ks] = key < p.N ? load_frag<Tr>(p.v + off + ks * Tr::kStep * E) : frag_t{};
    }
  }
  f32x16_t dkt[C::DB], dvt[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dkt[db] = dvt[db] = f32x16_t{};

  // Queries that can see any of the 128 keys: [first_query(kv0), end of the
  // last key's document). The (q head, query tile) iterations over them,
  // head-major, are split evenly between p.splits workgroups; this one takes
  // [it0, it1).
  const int q_end = doc_of(p.cu, p.ndocs, p.N, min(kv0 + 32 * kWaves - 1, p.N - 1)).end;
  const int qt0 = first_query(p, kv0) / C::QT;
  const int n_qt = (q_end - 1) / C::QT - qt0 + 1;
  const int n_it = n_qt * p.G;
  const int it0 = int(int64_t(n_it) * split / p.splits);
  const int it1 = int(int64_t(n_it) * (split + 1) / p.splits);
  auto head_of = [&](int it) { return kvh * p.G + it / n_qt; };
  auto qs_of = [&](int it) { return (qt0 + it % n_qt) * C::QT; };

  QTile<Tr, D> tile;
  if (it0 < it1) {
    tile.load(p, head_of(it0), qs_of(it0), tid);
    tile.store(smem, tid);
  }
  __syncthreads();
  // 64-row tiles: the next tile is loaded into registers during this one's
  // products; 32-row tiles (D = 128, no registers to spare): at its end
  constexpr bool kPrefetch = C::QT == 64;
  if (kPrefetch && it0 + 1 < it1) tile.load(p, head_of(it0 + 1), qs_of(it0 + 1), tid);

  for (int it = it0; it < it1; ++it) {
    const int qs = qs_of(it);
    const char* st = smem + ((it - it0) & 1) * C::STAGE;
    const char* qr = st;
    const char* dr = st + C::X_BYTES;
    const float* fl = reinterpret_cast<const float*>(st + 2 * C::X_BYTES);

    if (active && qs + C::QT - 1 >= kbd.w_lo_first && qs < w_de_last) {
      f32x16_t s[C::QB], dp[C::QB];
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) s[qb] = dp[qb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          const int row = qb * 32 + l32;
          const frag_t a = load_frag<Tr>(qr + row * C::F_STRIDE + (2 * ks + half) * 4);
          const frag_t b = load_frag<Tr>(dr + row * C::F_STRIDE + (2 * ks + half) * 4);
          s[qb] = mfma(a, kf[ks], s[qb]);
          dp[qb] = mfma(b, vf[ks], dp[qb]);
        }
      }
      const bool need_mask = (qs < kbd.w_lo_last) || (qs + C::QT > w_de_first);
      float pv[16 * C::QB], dsv[16 * C::QB];
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int qi = qb * 32 + 8 * r4 + 4 * half;  // first of 4 consecutive queries
          const float4 l4 = *reinterpret_cast<const float4*>(fl + qi);
          const float4 d4 = *reinterpret_cast<const float4*>(fl + C::QT + qi);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * r4 + j;
            float e = fast_exp2(fmaf(s[qb][r], p.scale_log2, -lv[j]));
            if (need_mask) {
              const int q = qs + qi + j;
              if (q < my_lo || q >= my_de) e = 0.f;
            }
            pv[qb * 16 + r] = e;
            dsv[qb * 16 + r] = e * (dp[qb][r] - dv4[j]);
          }
        }
      // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over the tile's queries)
#pragma unroll
      for (int st2 = 0; st2 < C::QS; ++st2) {
        const frag_t pf = make_frag<Tr>(&pv[st2 * Tr::kEpl]);
        const frag_t sf = make_frag<Tr>(&dsv[st2 * Tr::kEpl]);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int d = db * 32 + l32;
          const int qrow = (st2 >> 4) * 32 + acc_row(st2 & 15, half);
          const frag_t ad = load_frag<Tr>(dr + qrow * C::F_STRIDE + d * 4);
          const frag_t aq = load_frag<Tr>(qr + qrow * C::F_STRIDE + d * 4);
          dvt[db] = mfma(ad, pf, dvt[db]);
          dkt[db] = mfma(aq, sf, dkt[db]);
        }
      }
    }

    if (it + 1 < it1) {
      if (!kPrefetch) tile.load(p, head_of(it + 1), qs_of(it + 1), tid);
      tile.store(smem + ((it + 1 - it0) & 1) * C::STAGE, tid);
      if (kPrefetch && it + 2 < it1) tile.load(p, head_of(it + 2), qs_of(it + 2), tid);
    }
    __syncthreads();
  }

  // Epilogue: lane (key, half) holds d = 32 db + acc_row(r, half).
  if (p.splits > 1) {
    // fp32 partial sums, reduced in split order by dkdv_reduce_kernel
    if (active && key < p.N) {
      const int64_t off = ((int64_t(split) * p.N + key) * p.hk + kvh) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = db * 32 + 8 * r4 + 4 * half;
          *reinterpret_cast<f32x4_t*>(p.part_dk + off + d) =
              f32x4_t{dkt[db][4 * r4], dkt[db][4 * r4 + 1], dkt[db][4 * r4 + 2], dkt[db][4 * r4 + 3]};
          *reinterpret_cast<f32x4_t*>(p.part_dv + off + d) =
              f32x4_t{dvt[db][4 * r4], dvt[db][4 * r4 + 1], dvt[db][4 * r4 + 2], dvt[db][4 * r4 + 3]};
        }
    }
    return;
  }
  if (active && key < p.N) {
    constexpr int OE = kF32Out ? 4 : 2;
    const int64_t off = (int64_t(key) * p.hk + kvh) * D * OE;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * half;
        float kx[4], vx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kx[j] = dkt[db][4 * r4 + j] * p.scale;
          vx[j] = dvt[db][4 * r4 + j];
        }
        store4<kF32Out>(p.dk + off + d * OE, kx, p.accumulate);
        store4<kF32Out>(p.dv + off + d * OE, vx, p.accumulate);
      }
  }
}

// Sum of the split partials, in split order (deterministic), then the scale
// for dK and the output type. One thread per 4 consecutive elements.
template <bool kF32Out>
__global__ __launch_bounds__(kThreads) void dkdv_reduce_kernel(BwdParams p, int D) {
  const int64_t n4 = int64_t(p.N) * p.hk * D / 4;
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n4) return;
  const int64_t stride = int64_t(p.N) * p.hk * D;
  // bf16 inputs: undo the fp16 operand scales (BwdScales); fp32: dK's scale
  float mul_k = p.scale, mul_v = 1.f;
  if (p.absmax != nullptr) {
    const BwdScales sc = bwd_scales(p.absmax, p.scale);
    mul_k = sc.mul_dk;
    mul_v = sc.mul_dv;
  }
  float k[4] = {0.f, 0.f, 0.f, 0.f}, v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.splits; ++s) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p.part_dk + s * stride + 4 * i);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p.part_dv + s * stride + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      k[j] += a[j];
      v[j] += b[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    k[j] *= mul_k;
    v[j] *= mul_v;
  }
  constexpr int OE = kF32Out ? 4 : 2;
  store4<kF32Out>(p.dk + 4 * i * OE, k, p.accumulate);
  store4<kF32Out>(p.dv + 4 * i * OE, v, p.accumulate);
}

// ----------------------------------------------------------------------------
// 3. dQ (query-stationary)
// ----------------------------------------------------------------------------
// fp32
template <class Tr, int D>
struct QCfg {
  static_assert(Tr::kElem == 4, "fp32 kernel");
  static constexpr int E = Tr::kElem;
  static constexpr int KS = D / Tr::kStep;
  static constexpr int DB = D / 32;
  static constexpr int PV = BT / Tr::kStep;
  static constexpr int F_STRIDE = D * 4 + 16;
  static constexpr int X_BYTES = BT * F_STRIDE;
  static constexpr int STAGE = 2 * X_BYTES;  // K, V
  static constexpr int F_CH = BT * D * 4 / 16 / kThreads;
};

template <class Tr, int D>
struct KvTile {
  using C = QCfg<Tr, D>;
  static constexpr int NR = C::F_CH;
  u32x4_t xk[NR], xv[NR];

  __device__ __forceinline__ void load(const BwdParams& p, int kvh, int kv0, int tid) {
    const int64_t row_bytes = int64_t(p.hk) * D * C::E;
    const char* kb = p.k + int64_t(kvh) * D * C::E;
    const char* vb = p.v + int64_t(kvh) * D * C::E;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 4), col = c % (D / 4);
      const int key = kv0 + row;
      const bool ok = key < p.N;
      xk[i] = ok ? ld16(kb + key * row_bytes + col * 16) : u32x4_t{0, 0, 0, 0};
      xv[i] = ok ? ld16(vb + key * row_bytes + col * 16) : u32x4_t{0, 0, 0, 0};
    }
  }

  __device__ __forceinline__ void store(char* st, int tid) const {
    char* kr = st;
    char* vr = st + C::X_BYTES;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (D / 4), col = c % (D / 4);
      *reinterpret_cast<u32x4_t*>(kr + row * C::F_STRIDE + col * 16) = xk[i];
      *reinterpret_cast<u32x4_t*>(vr + row * C::F_STRIDE + col * 16) = xv[i];
    }
  }
};

template <class Tr, int D, bool kF32Out>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(BwdParams p) {
  using C = QCfg<Tr, D>;
  using frag_t = typename Tr::frag_t;
  constexpr int E = C::E;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int groups = p.G / p.Gw;
  const int kvh = blockIdx.y / groups, sub = blockIdx.y % groups;
  const int QW = kWaves / p.Gw;
  const int qtile = p.n_tiles - 1 - int(blockIdx.x);  // heaviest first
  const int wg_q0 = qtile * 32 * QW;
  const int wg_q1 = min(p.N, wg_q0 + 32 * QW);
  const int head = kvh * p.G + sub * p.Gw + (w % p.Gw);
  const int qbase = wg_q0 + (w / p.Gw) * 32;
  const bool active = qbase < p.N;
  const int wq_last = min(qbase + 31, p.N - 1);
  const int my_q = qbase + l32;
  const QueryBounds qbd(p, my_q, qbase, wq_last, active);
  const int my_ds = qbd.my_ds, my_hi = qbd.my_hi;
  const bool q_ok = my_q < p.N;
  const float my_lse2 = q_ok ? p.lse[int64_t(head) * p.N + my_q] * kLog2e : 0.f;
  const float my_dlt = q_ok ? p.delta[int64_t(head) * p.N + my_q] : 0.f;

  frag_t qf[C::KS], df[C::KS];
  {
    const int64_t off = (int64_t(my_q) * p.hq + head) * D * E + half * Tr::kEpl * E;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[ks] = q_ok ? load_frag<Tr>(p.q + off + ks * Tr::kStep * E) : frag_t{};
      df[ks] = q_ok ? load_frag<Tr>(p.dout + off + ks * Tr::kStep * E) : frag_t{};
    }
  }
  f32x16_t dqt[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dqt[db] = f32x16_t{};

  const int kv_begin = doc_of(p.cu, p.ndocs, p.N, wg_q0).start;
  const int kv_end = p.causal ? wg_q1 : doc_of(p.cu, p.ndocs, p.N, wg_q1 - 1).end;
  const int t0 = kv_begin / BT, t1 = (kv_end - 1) / BT;

  KvTile<Tr, D> tile;
  tile.load(p, kvh, t0 * BT, tid);
  tile.store(smem, tid);
  __syncthreads();
  if (t0 + 1 <= t1) tile.load(p, kvh, (t0 + 1) * BT, tid);

  for (int t = t0; t <= t1; ++t) {
    const int kv0 = t * BT;
    const char* st = smem + ((t - t0) & 1) * C::STAGE;
    const char* kr = st;
    const char* vr = st + C::X_BYTES;

    if (active && kv0 <= qbd.w_hi_last && kv0 + BT > qbd.w_ds_first) {
      f32x16_t s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = dp[kb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = kb * 32 + l32;
          const frag_t a = load_frag<Tr>(kr + row * C::F_STRIDE + (2 * ks + half) * 4);
          const frag_t b = load_frag<Tr>(vr + row * C::F_STRIDE + (2 * ks + half) * 4);
          s[kb] = mfma(a, qf[ks], s[kb]);
          dp[kb] = mfma(b, df[ks], dp[kb]);
        }
      }
      const bool need_mask = (kv0 + BT - 1 > qbd.w_hi_first) || (kv0 < qbd.w_ds_last);
      float dsv[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = fast_exp2(fmaf(s[kb][r], p.scale_log2, -my_lse2));
          if (need_mask) {
            const int key = kv0 + kb * 32 + acc_row(r, half);
            if (key > my_hi || key < my_ds) e = 0.f;
          }
          dsv[kb * 16 + r] = e * (dp[kb][r] - my_dlt);
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int st2 = 0; st2 < C::PV; ++st2) {
        const frag_t sf = make_frag<Tr>(&dsv[st2 * Tr::kEpl]);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int d = db * 32 + l32;
          const int krow = (st2 >> 4) * 32 + acc_row(st2 & 15, half);
          const frag_t a = load_frag<Tr>(kr + krow * C::F_STRIDE + d * 4);
          dqt[db] = mfma(a, sf, dqt[db]);
        }
      }
    }

    if (t + 1 <= t1) {
      tile.store(smem + ((t + 1 - t0) & 1) * C::STAGE, tid);
      if (t + 2 <= t1) tile.load(p, kvh, (t + 2) * BT, tid);
    }
    __syncthreads();
  }

  if (active && q_ok) {
    constexpr int OE = kF32Out ? 4 : 2;
    char* dst = p.dq + (int64_t(my_q) * p.hq + head) * D * OE;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * half;
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = dqt[db][4 * r4 + j] * p.scale;
        store4<kF32Out>(dst + d * OE, x, p.accumulate);
      }
  }
}


// ----------------------------------------------------------------------------
// bf16 kernels on row-major LDS tiles (lds_tile.hpp): every tile is copied by
// buffer_load ... lds (inline assembly, counted by explicit vmcnt waits) into
// a four-stage ring, three tiles ahead, and the transposed operands (Q^T,
// dO^T, K^T) are read with ds_read_b64_tr_b16 instead of being stored twice.
// One barrier per tile; a stage is refilled only after the tile's LDS reads.
// ----------------------------------------------------------------------------
template <int D>
struct DqBf {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TB = TileFmt<D>::kBytes;
  static constexpr int STAGE = 2 * TB;  // K, V
  static constexpr int NSTAGE = 4;
  static constexpr int LOADS = 2 * tile_loads<D, kThreads>();
};

template <int D, bool kF32Out>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void dq_bf16_kernel(BwdParams p) {
  using C = DqBf<D>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::NSTAGE * C::STAGE];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int groups = p.G / p.Gw;
  const int kvh = blockIdx.y / groups, sub = blockIdx.y % groups;
  const int QW = C::kWaves / p.Gw;
  // heaviest first: by position in the sequence, or with a few packed
  // documents by position in the document
  const int qtile = (p.cu != nullptr && p.causal && p.ndocs <= 64)
                        ? uniform(tile_by_work_rank(p.cu, p.ndocs, p.N, 32 * QW, p.n_tiles, int(blockIdx.x)))
                        : p.n_tiles - 1 - int(blockIdx.x);
  const int wg_q0 = qtile * 32 * QW;
  const int wg_q1 = min(p.N, wg_q0 + 32 * QW);
  const int head = kvh * p.G + sub * p.Gw + (w % p.Gw);
  const int qbase = wg_q0 + (w / p.Gw) * 32;
  const bool active = qbase < p.N;
  const int wq_last = min(qbase + 31, p.N - 1);
  const int my_q = qbase + l32;
  const bool q_ok = my_q < p.N;
  const QueryBounds qbd(p, my_q, qbase, wq_last, active);
  const int my_ds = qbd.my_ds, my_hi = qbd.my_hi;
  const BwdScales sc = bwd_scales(p.absmax, p.scale);
  const float my_lse2 = q_ok ? p.lse2[int64_t(head) * p.N + my_q] : 0.f;
  const float my_dlt = q_ok ? p.delta[int64_t(head) * p.N + my_q] : 0.f;

  bf16x8_t qf[C::KS], df[C::KS];
  {
    const int64_t off = (int64_t(my_q) * p.hq + head) * D * 2 + half * 16;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[ks] = q_ok ? *reinterpret_cast<const bf16x8_t*>(p.q16 + off + ks * 32) : bf16x8_t{};
      df[ks] = q_ok ? *reinterpret_cast<const bf16x8_t*>(p.do16 + off + ks * 32) : bf16x8_t{};
    }
  }
  f32x16_t dqt[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dqt[db] = f32x16_t{};

  const int kv_begin = doc_of(p.cu, p.ndocs, p.N, wg_q0).start;
  const int kv_end = p.causal ? wg_q1 : doc_of(p.cu, p.ndocs, p.N, wg_q1 - 1).end;
  const int t0 = kv_begin / BT, t1 = (kv_end - 1) / BT;
  const uint32_t kv_row = uint32_t(p.hk) * D * 2;

  auto issue = [&](int t) {
    lds_char* st = smem + ((t - t0) % C::NSTAGE) * C::STAGE;
    const int kv0 = t * BT;
    const uint32_t bytes = uint32_t(min(BT, p.N - kv0)) * kv_row;
    const int64_t off = (int64_t(kv0) * p.hk + kvh) * D * 2;
    issue_tile<D, C::kThreads, 64, true>(make_rsrc_uniform(p.k16 + off, bytes), kv_row, st, tid);
    issue_tile<D, C::kThreads, 64, true>(make_rsrc_uniform(p.v16 + off, bytes), kv_row, st + C::TB, tid);
  };
  // The tile copies are inline assembly, unknown to the compiler: its own
  // loads (Q, dO, lse, delta rows) are complete here, so it adds no wait of
  // its own later that would also drain the copies in flight.
  wait_vmcnt<0>();
  issue(t0);
  if (t0 + 1 <= t1) issue(t0 + 1);
  if (t0 + 2 <= t1) issue(t0 + 2);

  for (int t = t0; t <= t1; ++t) {
    if (t + 2 <= t1) wait_vmcnt<2 * C::LOADS>(); else if (t + 1 <= t1) wait_vmcnt<C::LOADS>(); else wait_vmcnt<0>();
    __syncthreads();
    const int kv0 = t * BT;
    const lds_char* kr = smem + ((t - t0) % C::NSTAGE) * C::STAGE;
    const lds_char* vr = kr + C::TB;

    if (active && kv0 <= qbd.w_hi_last && kv0 + BT > qbd.w_ds_first) {
      const bool need_mask = (kv0 + BT - 1 > qbd.w_hi_first) || (kv0 < qbd.w_ds_last);
      f32x16_t s[2] = {f32x16_t{}, f32x16_t{}}, dp[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = mfma_f16(frag_rows<D>(kr, kb * 32 + l32, ks * 16, half), qf[ks], s[kb]);
          dp[kb] = mfma_f16(frag_rows<D>(vr, kb * 32 + l32, ks * 16, half), df[ks], dp[kb]);
        }
      // masked scores become -inf (their exponentials exact zeros) in a loop
      // of their own, so the exponentials below are one straight run
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int k = kv0 + kb * 32 + acc_row(r, half);
            if (k > my_hi || k < my_ds) s[kb][r] = -INFINITY;
          }
      }
      float dsv[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // e = P * 2^15, dsv = dS * 2^eds (see BwdScales)
          const float e = fast_exp2(fmaf(s[kb][r], sc.c_s, -my_lse2));
          dsv[kb * 16 + r] = e * fmaf(dp[kb][r], sc.kd, -my_dlt);
        }
      // dQ^T += K^T dS^T, K^T read transposed from the row-major K tile
#pragma unroll
      for (int st2 = 0; st2 < BT / 16; ++st2) {
        const bf16x8_t sf = make_frag_f16(&dsv[st2 * 8]);
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          dqt[db] = mfma_f16(frag_cols_tr<D>(kr, st2 * 16, db * 32, lane), sf, dqt[db]);
      }
    }
    if (t + 3 <= t1) issue(t + 3);
  }

  if (active && q_ok) {
    constexpr int OE = kF32Out ? 4 : 2;
    char* dst = p.dq + (int64_t(my_q) * p.hq + head) * D * OE;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * half;
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = dqt[db][4 * r4 + j] * sc.mul_dq;
        store4<kF32Out>(dst + d * OE, x, p.accumulate);
      }
  }
}

template <class Tr, int D, bool kF32Out>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, void* workspace, const AttnDesc& d, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const char*>(q);
  p.k = static_cast<const char*>(k);
  p.v = static_cast<const char*>(v);
  p.o = static_cast<const char*>(o);
  p.dout = static_cast<const char*>(dout);
  p.lse = lse;
  p.dq = static_cast<char*>(dq);
  p.dk = static_cast<char*>(dk);
  p.dv = static_cast<char*>(dv);
  const BwdWorkspace wl = bwd_workspace_layout(d);
  p.delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.delta);
  p.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.lse2);
  p.splits = bwd_dkdv_splits(d);
  char* ws = static_cast<char*>(workspace);
  const bool half_ops = Tr::kElem == 2;  // bf16 inputs: fp16 operand copies (BwdScales)
  p.absmax = half_ops ? reinterpret_cast<uint32_t*>(ws + wl.absmax) : nullptr;
  p.q16 = half_ops ? ws + wl.q16 : nullptr;
  p.do16 = half_ops ? ws + wl.do16 : nullptr;
  p.k16 = half_ops ? ws + wl.k16 : nullptr;
  p.v16 = half_ops ? ws + wl.v16 : nullptr;
  p.part_dk = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.part);
  p.part_dv = p.part_dk + (p.splits > 1 ? size_t(p.splits) * d.N * d.hk * d.D : 0);
  p.cu = d.cu;
  p.ndocs = d.ndocs;
  p.N = static_cast<int>(d.N);
  p.hq = d.hq;
  p.hk = d.hk;
  p.G = d.hq / d.hk;
  p.Gw = std::gcd(p.G, kWaves);
  p.scale = d.scale;
  p.scale_log2 = d.scale * kLog2e;
  p.causal = d.causal;
  p.accumulate = d.accumulate;

  const int64_t rows = d.N * d.hq;
  const int64_t rows_per_block = kThreads / (D * Tr::kElem / 16);
  const int64_t row_blocks = (rows + rows_per_block - 1) / rows_per_block;
  hipError_t e;
  if constexpr (Tr::kElem == 2) {
    // delta, lse2 and the maxima, then the scaled fp16 copies; a few
    // thousand workgroups loop over the rows (one atomic max per workgroup)
    const unsigned prep_blocks = static_cast<unsigned>(std::min<int64_t>(row_blocks, 4096));
    absmax_init_kernel<<<1, 64, 0, stream>>>(p.absmax);
    prep_bf16_kernel<D><<<dim3(prep_blocks), kThreads, 0, stream>>>(p);
    convert_bf16_kernel<D><<<dim3(4096), kThreads, 0, stream>>>(p);
  } else {
    delta_kernel<Tr, D><<<dim3(static_cast<unsigned>(row_blocks)), kThreads, 0, stream>>>(p);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  if constexpr (Tr::kElem == 2)
    e = launch_dkdv_bf16<D, kF32Out>(p, p.splits, d.hk, stream);
  else {
    p.n_tiles = static_cast<int>((d.N + kKeysPerWg - 1) / kKeysPerWg);
    dkdv_kernel<Tr, D, kF32Out><<<dim3(p.n_tiles * p.splits, d.hk), kThreads, 0, stream>>>(p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (p.splits > 1) {
    const int64_t n4 = d.N * d.hk * D / 4;
    dkdv_reduce_kernel<kF32Out><<<dim3(static_cast<unsigned>((n4 + kThreads - 1) / kThreads)), kThreads, 0, stream>>>(
        p, D);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  if constexpr (Tr::kElem == 2) {
    p.Gw = std::gcd(p.G, DqBf<D>::kWaves);
    const int rows_per_wg = 32 * (DqBf<D>::kWaves / p.Gw);
    p.n_tiles = static_cast<int>((d.N + rows_per_wg - 1) / rows_per_wg);
    dq_bf16_kernel<D, kF32Out><<<dim3(p.n_tiles, d.hk * (p.G / p.Gw)), DqBf<D>::kThreads, 0, stream>>>(p);
  } else {
    const int rows_per_wg = 32 * (kWaves / p.Gw);
    p.n_tiles = static_cast<int>((d.N + rows_per_wg - 1) / rows_per_wg);
    dq_kernel<Tr, D, kF32Out><<<dim3(p.n_tiles, d.hk * (p.G / p.Gw)), kThreads, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, void* workspace, const AttnDesc& d,
                           uly_dtype grad_dt, hipStream_t stream) {
  if (d.dt == ULY_BF16) {
    if (grad_dt == ULY_F32)
      return d.D == 128 ? launch<TrBF16, 128, true>(q, k, v, o, dout, lse, dq, dk, dv, workspace, d, stream)
                        : launch<TrBF16, 64, true>(q, k, v, o, dout, lse, dq, dk, dv, workspace, d, stream);
    return d.D == 128 ? launch<TrBF16, 128, false>(q, k, v, o, dout, lse, dq, dk, dv, workspace, d, stream)
                      : launch<TrBF16, 64, false>(q, k, v, o, dout, lse, dq, dk, dv, workspace, d, stream);
  }
  return d.D == 128 ? launch<TrF32, 128, true>(q, k, v, o, dout, lse, dq, dk, dv, workspace, d, stream)
                    : launch<TrF32, 64, true>(q, k, v, o, dout, lse, dq, dk, dv, workspace, d, stream);
}

}  // namespace uly
