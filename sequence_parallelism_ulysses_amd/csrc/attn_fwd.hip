// Causal (or document-only masked) GQA / packed-document attention forward
// for one head group.
//
// Exact softmax attention computed in key tiles with an online (running-max)
// softmax, so the N x N score matrix is never stored ("Ulysses Sequence
// Parallelism: Training with Million-Token Contexts": tiled attention keeps
// memory linear while the compute stays quadratic; "Snowflake's Ulysses trick
// ...", second paragraph: each GPU runs standard attention over the full
// sequence for its heads).
//
// Two kernels share the decomposition: the Gw = gcd(G, waves) q heads of
// one kv head that share K/V are folded into one workgroup, so each K/V tile
// read from HBM/L2 serves Gw heads; every wave owns 32 query rows of one q
// head, held in registers as the MFMA B operand; K/V tiles hold 64 keys;
// workgroups are launched heaviest causal row-tile first.
//   - fp32 (attn_fwd_kernel): 4 waves, v_mfma_f32_32x32x2f32, tiles staged
//     through registers into a double-buffered LDS pair, one barrier per tile;
//   - bf16 (attn_fwd_bf16_kernel): 8 waves (two per SIMD, running half a tile
//     apart), v_mfma_f32_32x32x16_bf16, tiles copied global -> LDS by buffer
//     loads into a four-stage ring, V^T read with ds_read_b64_tr_b16.
//
// Per wave and tile the math runs transposed, S^T = K Q^T, so that each lane
// owns one query column: the row max and row sum of the softmax are per-lane
// reductions plus one v_permlane32_swap between the two half-waves. The
// probabilities are then already laid out as the B operand of O^T += V^T P^T.
//
// Masking (key j, query i): doc_start(i) <= j <= hi(i), with hi(i) = i for
// causal attention and the last token of i's document otherwise. Only tiles
// past some row's hi (the diagonal tile when causal) and tiles crossing a
// document start are masked element-wise; tiles that no row of a wave can see
// are skipped by that wave.
#include <cmath>
#include <numeric>

#include "common.hpp"
#include "internal.hpp"
#include "lds_tile.hpp"

namespace uly {
namespace {

constexpr int BN = 64;  // keys per tile

struct FwdParams {
  const char* q;
  const char* k;
  const char* v;
  char* o;
  float* lse;
  const int32_t* cu;
  int ndocs;
  int N, hq, hk, G, Gw;
  int n_qtiles;
  int causal;
  float scale_log2;
};

// Sequence-sharded sources read in place (the bf16 kernel's shard mode): the
// token n of a head group lives in shard n / T at row n % T, its heads after
// q_head0 / kv_head0. With T a multiple of 64 a wave's 32 query rows and a
// 64-key tile each lie in one shard.
struct ShardSrc {
  const char* q[ULY_MAX_P];
  const char* k[ULY_MAX_P];
  const char* v[ULY_MAX_P];
  int T;
  int q_row;     // bytes of one shard token of Q (all Hq heads)
  int kv_row;    // bytes of one shard token of K or V (all Hkv heads)
  int q_head0;   // first query head of the group in a shard token
  int kv_head0;  // first kv head of the group
};

// The fp32 kernel: 4 waves of 32 query rows.
template <class Tr, int D>
struct FwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int E = Tr::kElem;
  static constexpr int QB = 1;  // 32-row blocks per wave
  static constexpr int RW = 32 * QB;
  static constexpr int KS = D / Tr::kStep;  // MFMA steps over D
  static constexpr int DB = D / 32;         // 32-wide blocks of D
  static constexpr int PV = BN / Tr::kStep; // MFMA steps over the keys of a tile
  static constexpr int K_STRIDE = D * E + 16;  // rows padded by 16 bytes
  static constexpr int V_STRIDE = D * E + 16;
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int V_BYTES = BN * V_STRIDE;
  static constexpr int CPR = D * E / 16;            // 16-byte chunks per row
  static constexpr int K_CH = BN * CPR / kThreads;  // chunks per thread
  static_assert(BN * CPR % kThreads == 0, "tile must split evenly");
};

template <class Tr, int D>
struct Tile {
  using C = FwdCfg<Tr, D>;
  static constexpr int kThreads = C::kThreads;
  u32x4_t k[C::K_CH];
  u32x4_t v[C::K_CH];

  __device__ __forceinline__ void load(const FwdParams& p, int kvh, int kv0, int tid) {
    const int64_t row_bytes = int64_t(p.hk) * D * C::E;
    const char* kb = p.k + int64_t(kvh) * D * C::E;
    const char* vb = p.v + int64_t(kvh) * D * C::E;
#pragma unroll
    for (int i = 0; i < C::K_CH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / C::CPR, col = c % C::CPR;
      const int key = kv0 + row;
      k[i] = key < p.N ? *reinterpret_cast<const u32x4_t*>(kb + key * row_bytes + col * 16) : u32x4_t{0, 0, 0, 0};
      v[i] = key < p.N ? *reinterpret_cast<const u32x4_t*>(vb + key * row_bytes + col * 16) : u32x4_t{0, 0, 0, 0};
    }
  }

  __device__ __forceinline__ void store(char* lk, char* lv, int tid) const {
#pragma unroll
    for (int i = 0; i < C::K_CH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / C::CPR, col = c % C::CPR;
      *reinterpret_cast<u32x4_t*>(lk + row * C::K_STRIDE + col * 16) = k[i];
      *reinterpret_cast<u32x4_t*>(lv + row * C::V_STRIDE + col * 16) = v[i];
    }
  }
};

template <class Tr, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(FwdCfg<Tr, D>::kThreads, FwdCfg<Tr, D>::kThreads),
                          amdgpu_waves_per_eu(FwdCfg<Tr, D>::kWaves / 4, FwdCfg<Tr, D>::kWaves / 4)))
void attn_fwd_kernel(FwdParams p) {
  using C = FwdCfg<Tr, D>;
  using frag_t = typename Tr::frag_t;
  constexpr int E = C::E, QB = C::QB, RW = C::RW, kWaves = C::kWaves;
  __shared__ __attribute__((aligned(16))) char smem[2 * (C::K_BYTES + C::V_BYTES)];

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int groups = p.G / p.Gw;
  const int kvh = blockIdx.y / groups, sub = blockIdx.y % groups;
  const int QW = kWaves / p.Gw;
  const int qtile = p.n_qtiles - 1 - int(blockIdx.x);  // heaviest first
  const int wg_q0 = qtile * RW * QW;
  const int wg_q1 = min(p.N, wg_q0 + RW * QW);
  const int head = kvh * p.G + sub * p.Gw + (w % p.Gw);
  const int qbase = wg_q0 + (w / p.Gw) * RW;
  const bool active = qbase < p.N;
  const int wq_last = min(qbase + RW - 1, p.N - 1);

  // Query rows of this lane, their document starts, and the wave's bounds.
  // Row i sees keys [doc start, hi(i)]: hi(i) = i when causal, else the
  // last token of its document.
  int my_q[QB], my_ds[QB], my_hi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    my_q[qb] = qbase + qb * 32 + l32;
    const DocSpan dsp = doc_of(p.cu, p.ndocs, p.N, min(my_q[qb], p.N - 1));
    my_ds[qb] = dsp.start;
    my_hi[qb] = p.causal ? my_q[qb] : dsp.end - 1;
  }
  const DocSpan w_doc_first = doc_of(p.cu, p.ndocs, p.N, min(qbase, p.N - 1));
  const DocSpan w_doc_last = doc_of(p.cu, p.ndocs, p.N, wq_last);
  const int w_ds_first = active ? w_doc_first.start : 0;
  const int w_ds_last = w_doc_last.start;
  const int w_hi_first = p.causal ? qbase : w_doc_first.end - 1;
  const int w_hi_last = p.causal ? wq_last : w_doc_last.end - 1;

  // Q fragments (B operand of S^T = K Q^T), zero past N.
  frag_t qf[QB][C::KS];
  const int64_t q_row = int64_t(p.hq) * D * E;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const char* src = p.q + int64_t(my_q[qb]) * q_row + int64_t(head) * D * E + half * Tr::kEpl * E;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[qb][ks] = my_q[qb] < p.N ? load_frag<Tr>(src + ks * Tr::kStep * E) : frag_t{};
  }

  f32x16_t acc_o[C::DB][QB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc_o[db][qb] = f32x16_t{};
  }

  const int kv_begin = doc_of(p.cu, p.ndocs, p.N, wg_q0).start;
  const int kv_end = p.causal ? wg_q1 : doc_of(p.cu, p.ndocs, p.N, wg_q1 - 1).end;
  const int t0 = kv_begin / BN, t1 = (kv_end - 1) / BN;

  Tile<Tr, D> tile;
  tile.load(p, kvh, t0 * BN, tid);
  tile.store(smem, smem + C::K_BYTES, tid);
  __syncthreads();
  if (t0 + 1 <= t1) tile.load(p, kvh, (t0 + 1) * BN, tid);

  for (int t = t0; t <= t1; ++t) {
    const int kv0 = t * BN;
    const char* lk = smem + ((t - t0) & 1) * (C::K_BYTES + C::V_BYTES);
    const char* lv = lk + C::K_BYTES;

    if (active && kv0 <= w_hi_last && kv0 + BN > w_ds_first) {
      // element-wise mask only on tiles past some row's last visible key (the
      // diagonal tile when causal) and tiles crossing a document start
      const bool need_mask = __builtin_expect(kv0 + BN - 1 > w_hi_first || kv0 < w_ds_last, 0);
      // S^T tile: keys (2 blocks of 32) x this wave's query columns.
      f32x16_t s[2][QB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const frag_t a = load_frag<Tr>(lk + (kb * 32 + l32) * C::K_STRIDE + (ks * Tr::kStep + half * Tr::kEpl) * E);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma(a, qf[qb][ks], s[kb][qb]);
        }
      }

      frag_t pf[QB][C::PV];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kv0 + kb * 32 + acc_row(r, half);
              if (key > my_hi[qb] || key < my_ds[qb]) s[kb][qb][r] = -INFINITY;
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][qb][r]);
        mt = xhalf_max(mt) * p.scale_log2;
        // raise the running max only when the tile's max exceeds it by > 2^8
        const bool grow = mt > m[qb] + kRescaleLog2;
        if (wave_any(grow)) {
          // lanes that do not grow keep their max (alpha 1, also when it is still -inf);
          // a growing lane whose max was -inf gets alpha 0
          const float alpha = grow ? fast_exp2(m[qb] - mt) : 1.f;
          m[qb] = grow ? mt : m[qb];
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) acc_o[db][qb] *= alpha;
        }
        const float m_use = m[qb] == -INFINITY ? 0.f : m[qb];
        float pv[32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(s[kb][qb][r], p.scale_log2, -m_use));
            pv[kb * 16 + r] = e;
            l[qb] += e;
          }
#pragma unroll
        for (int st = 0; st < C::PV; ++st) pf[qb][st] = make_frag<Tr>(&pv[st * Tr::kEpl]);
      }

      // O^T += V^T P^T
#pragma unroll
      for (int st = 0; st < C::PV; ++st) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int key = (st >> 4) * 32 + acc_row(st & 15, half);
          const frag_t a = load_frag<Tr>(lv + key * C::V_STRIDE + (db * 32 + l32) * E);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc_o[db][qb] = mfma(a, pf[qb][st], acc_o[db][qb]);
        }
      }
    }

    if (t + 1 <= t1) {
      char* nk = smem + ((t + 1 - t0) & 1) * (C::K_BYTES + C::V_BYTES);
      tile.store(nk, nk + C::K_BYTES, tid);
      if (t + 2 <= t1) tile.load(p, kvh, (t + 2) * BN, tid);
    }
    __syncthreads();
  }

  // Epilogue: normalise, write O (rounded to the I/O type) and the natural-log LSE.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lsum = xhalf_sum(l[qb]);
    const int q = my_q[qb];
    if (!active || q >= p.N) continue;
    const float inv = 1.f / lsum;
    char* dst = p.o + int64_t(q) * q_row + int64_t(head) * D * E;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * half;
        const float x0 = acc_o[db][qb][4 * r4 + 0] * inv, x1 = acc_o[db][qb][4 * r4 + 1] * inv;
        const float x2 = acc_o[db][qb][4 * r4 + 2] * inv, x3 = acc_o[db][qb][4 * r4 + 3] * inv;
        if constexpr (E == 2) {
          *reinterpret_cast<u32x2_t*>(dst + d * E) = u32x2_t{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        } else {
          *reinterpret_cast<u32x4_t*>(dst + d * E) =
              u32x4_t{__float_as_uint(x0), __float_as_uint(x1), __float_as_uint(x2), __float_as_uint(x3)};
        }
      }
    if (half == 0) p.lse[int64_t(head) * p.N + q] = (m[qb] + log2f(lsum)) * kLn2;
  }
}


// ---------------------------------------------------------------------------
// bf16 kernel: K and V tiles stay row-major in LDS (swizzled, see
// lds_tile.hpp), filled by asynchronous buffer loads into a four-stage ring;
// V^T operands come from ds_read_b64_tr_b16. No register staging, no
// transposing stores.
//
// The two waves of a SIMD (w and w + 4) run half an iteration apart: each
// key tile takes two phases separated by barriers, and in each phase one of
// them issues the products S = K Q^T while the other runs the softmax and
// O += V P of the tile before, so the matrix unit has work while the other
// wave's exponentials run.
// ---------------------------------------------------------------------------
template <int D>
struct FwdBf {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int KS = D / 16;  // MFMA steps over D
  static constexpr int DB = D / 32;  // 32-wide blocks of D
  static constexpr int TB = TileFmt<D>::kBytes;
  static constexpr int STAGE = 2 * TB;  // K tile, V tile
  static constexpr int NSTAGE = 4;
  static constexpr int kCopiers = kThreads / 2;  // one group of four waves copies one tensor
  static constexpr int LOADS = tile_loads<D, kCopiers>();  // per copying lane per stage
};

template <int D, bool kShards>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(FwdParams p, ShardSrc sh) {
  using C = FwdBf<D>;
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
                        ? uniform(tile_by_work_rank(p.cu, p.ndocs, p.N, 32 * QW, p.n_qtiles, int(blockIdx.x)))
                        : p.n_qtiles - 1 - int(blockIdx.x);
  const int wg_q0 = qtile * 32 * QW;
  const int wg_q1 = min(p.N, wg_q0 + 32 * QW);
  const int head = kvh * p.G + sub * p.Gw + (w % p.Gw);
  const int qbase = wg_q0 + (w / p.Gw) * 32;
  const bool active = qbase < p.N;
  const int wq_last = min(qbase + 31, p.N - 1);
  const int my_q = qbase + l32;
  // Row i sees keys [doc start, hi(i)]: hi(i) = i when causal, else the
  // last token of its document.
  const DocSpan my_doc = doc_of(p.cu, p.ndocs, p.N, min(my_q, p.N - 1));
  const int my_ds = my_doc.start;
  const int my_hi = p.causal ? my_q : my_doc.end - 1;
  const DocSpan w_doc_first = doc_of(p.cu, p.ndocs, p.N, min(qbase, p.N - 1));
  const DocSpan w_doc_last = doc_of(p.cu, p.ndocs, p.N, wq_last);
  const int w_ds_first = active ? w_doc_first.start : 0;
  const int w_ds_last = w_doc_last.start;
  const int w_hi_first = p.causal ? qbase : w_doc_first.end - 1;
  const int w_hi_last = p.causal ? wq_last : w_doc_last.end - 1;

  // Q fragments (B operand of S^T = K Q^T), zero past N.
  bf16x8_t qf[C::KS];
  const int64_t q_row = int64_t(p.hq) * D * 2;
  {
    const char* src;
    if constexpr (kShards) {
      // the wave's 32 rows lie in one shard (T is a multiple of 64)
      const int j = uniform(min(qbase, p.N - 1) / sh.T);
      const int t = my_q - j * sh.T;
      src = sh.q[j] + int64_t(t) * sh.q_row + int64_t(sh.q_head0 + head) * D * 2 + half * 16;
    } else {
      src = p.q + int64_t(my_q) * q_row + int64_t(head) * D * 2 + half * 16;
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[ks] = my_q < p.N ? *reinterpret_cast<const bf16x8_t*>(src + ks * 32) : bf16x8_t{};
  }

  f32x16_t acc_o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc_o[db] = f32x16_t{};
  float m = -INFINITY, l = 0.f;
  RowFragOffsets<D> ko;
  TrFragOffsets<D> vo;
  ko.init(lane);
  vo.init(lane);

  const int kv_begin = doc_of(p.cu, p.ndocs, p.N, wg_q0).start;
  const int kv_end = p.causal ? wg_q1 : doc_of(p.cu, p.ndocs, p.N, wg_q1 - 1).end;
  const int t0 = kv_begin / BN, t1 = (kv_end - 1) / BN;
  const uint32_t kv_row = uint32_t(p.hk) * D * 2;

  // Group A (waves 0-3) runs tile t's products in the first phase of
  // iteration t and its softmax in the second; group B (waves 4-7) the
  // products in the second phase and the softmax in the first phase of
  // iteration t+1. Each group copies one tensor of tile t+3 after its
  // products (A the K tile, B the V tile), where the copies' stall at the
  // address unit costs least; the copies are inline-assembly DMA, so that
  // the compiler does not make transposed LDS reads wait for them, and each
  // group waits for its own before the first barrier of an iteration.
  const bool grp_b = w >= C::kWaves / 2;
  const int gtid = tid & (C::kCopiers - 1);
  auto issue = [&](int t, bool v_tile) {
    lds_char* st = smem + ((t - t0) % C::NSTAGE) * C::STAGE;
    const int kv0 = t * BN;
    if constexpr (kShards) {
      // the tile's 64 keys lie in shard j (T is a multiple of 64); rows are a
      // shard token apart, and the resource ends after the last valid row's head
      const int j = kv0 / sh.T, r0 = kv0 - j * sh.T;
      const char* base = (v_tile ? sh.v[j] : sh.k[j]) + int64_t(r0) * sh.kv_row + int64_t(sh.kv_head0 + kvh) * D * 2;
      const uint32_t bytes = uint32_t(min(BN, p.N - kv0) - 1) * uint32_t(sh.kv_row) + D * 2;
      issue_tile<D, C::kCopiers, 64, true>(make_rsrc_uniform(base, bytes), uint32_t(sh.kv_row),
                                           st + (v_tile ? C::TB : 0), gtid);
    } else {
      const uint32_t bytes = uint32_t(min(BN, p.N - kv0)) * kv_row;
      const int64_t off = (int64_t(kv0) * p.hk + kvh) * D * 2;
      issue_tile<D, C::kCopiers, 64, true>(make_rsrc_uniform((v_tile ? p.v : p.k) + off, bytes), kv_row,
                                           st + (v_tile ? C::TB : 0), gtid);
    }
  };
  // tile t must have landed; this group's copies of up to two later tiles may be in flight
  auto wait_tile = [&](int t) {
    const int ahead = min(2, t1 - t);
    if (ahead == 2) wait_vmcnt<2 * C::LOADS>(); else if (ahead == 1) wait_vmcnt<C::LOADS>(); else wait_vmcnt<0>();
  };
  auto sees = [&](int t) {
    const int kv0 = t * BN;
    return active && kv0 <= w_hi_last && kv0 + BN > w_ds_first;
  };
  auto compute_s = [&](int t, f32x16_t (&s)[2]) {
    const lds_char* lk = smem + ((t - t0) % C::NSTAGE) * C::STAGE;
    s[0] = f32x16_t{};
    s[1] = f32x16_t{};
    // all K reads of the tile go out before the first product, so the
    // products run back to back rather than each waiting on its own read
    bf16x8_t kf[C::KS][2];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const lds_char* ka = lds_base(lk, ko.off[ks]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[ks][kb] = frag_rows_at<D>(ka, kb * 64 * D);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma(kf[ks][kb], qf[ks], s[kb]);
  };

  // mask, online softmax and O^T += V^T P^T for tile t, S(t) in s
  auto softmax_pv = [&](int t, f32x16_t (&s)[2]) {
    const int kv0 = t * BN;
    const lds_char* lv = smem + ((t - t0) % C::NSTAGE) * C::STAGE + C::TB;
    // element-wise mask only on tiles past some row's last visible key (the
    // diagonal tile when causal) and tiles crossing a document start
    const bool need_mask = kv0 + BN - 1 > w_hi_first || kv0 < w_ds_last;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + acc_row(r, half);
          if (key > my_hi || key < my_ds) s[kb][r] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = xhalf_max(mt) * p.scale_log2;
    // raise the running max only when the tile's max exceeds it by > 2^8
    const bool grow = mt > m + kRescaleLog2;
    if (wave_any(grow)) {
      const float alpha = grow ? fast_exp2(m - mt) : 1.f;  // 0 when m was -inf
      m = grow ? mt : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) acc_o[db] *= alpha;
    }
    const float m_use = m == -INFINITY ? 0.f : m;
    float pv[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(s[kb][r], p.scale_log2, -m_use));
        pv[kb * 16 + r] = e;
        l += e;
      }
    // O^T += V^T P^T, 16 keys per step; V^T read transposed from the row-major tile
    const lds_char* va[2][C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      va[0][db] = lds_base(lv, vo.off[0][db]);
      va[1][db] = lds_base(lv, vo.off[1][db]);
    }
#pragma unroll
    for (int st = 0; st < BN / 16; ++st) {
      const bf16x8_t pf = make_frag<TrBF16>(&pv[st * 8]);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        acc_o[db] = mfma(frag_tr2(va[0][db], va[1][db], st * 32 * D), pf, acc_o[db]);
    }
  };

  // One loop per group (the barrier counts match), so that each keeps only
  // its own values in registers.
  f32x16_t s[2];
  // The compiler's own loads (Q rows, document offsets) are complete before
  // the first copy, so it adds no wait of its own later (at the first masked
  // tile) that would also drain the copies in flight, which it cannot see.
  wait_vmcnt<0>();
  for (int i = 0; i < 3; ++i)
    if (t0 + i <= t1) issue(t0 + i, grp_b);
  if (!grp_b) {
    for (int t = t0; t <= t1 + 1; ++t) {
      if (t <= t1) wait_tile(t);
      __syncthreads();
      if (t <= t1 && sees(t)) compute_s(t, s);
      // K of tile t-1 was last read by group B's products in the previous
      // iteration's second phase
      if (t + 3 <= t1) issue(t + 3, false);
      __syncthreads();
      if (t <= t1 && sees(t)) softmax_pv(t, s);
    }
  } else {
    for (int t = t0; t <= t1 + 1; ++t) {
      if (t <= t1) wait_tile(t);
      __syncthreads();
      if (t - 1 >= t0 && sees(t - 1)) softmax_pv(t - 1, s);
      __syncthreads();
      if (t <= t1 && sees(t)) compute_s(t, s);
      // V of tile t-1 was last read by this group's softmax of it, before
      // the second barrier
      if (t + 3 <= t1) issue(t + 3, true);
    }
  }

  const float lsum = xhalf_sum(l);
  if (active && my_q < p.N) {
    const float inv = 1.f / lsum;
    char* dst = p.o + int64_t(my_q) * q_row + int64_t(head) * D * 2;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * half;
        *reinterpret_cast<u32x2_t*>(dst + d * 2) =
            u32x2_t{pack_bf16x2(acc_o[db][4 * r4] * inv, acc_o[db][4 * r4 + 1] * inv),
                    pack_bf16x2(acc_o[db][4 * r4 + 2] * inv, acc_o[db][4 * r4 + 3] * inv)};
      }
    if (half == 0) p.lse[int64_t(head) * p.N + my_q] = (m + log2f(lsum)) * kLn2;
  }
}

template <int D>
hipError_t launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, const AttnDesc& d,
                       hipStream_t stream, const ShardSrc* shards = nullptr) {
  using C = FwdBf<D>;
  FwdParams p;
  p.q = static_cast<const char*>(q);
  p.k = static_cast<const char*>(k);
  p.v = static_cast<const char*>(v);
  p.o = static_cast<char*>(o);
  p.lse = lse;
  p.cu = d.cu;
  p.ndocs = d.ndocs;
  p.N = static_cast<int>(d.N);
  p.hq = d.hq;
  p.hk = d.hk;
  p.G = d.hq / d.hk;
  p.Gw = std::gcd(p.G, C::kWaves);
  const int rows = 32 * (C::kWaves / p.Gw);
  p.n_qtiles = static_cast<int>((d.N + rows - 1) / rows);
  p.scale_log2 = d.scale * kLog2e;
  p.causal = d.causal;
  dim3 grid(p.n_qtiles, d.hk * (p.G / p.Gw));
  if (shards)
    attn_fwd_bf16_kernel<D, true><<<grid, C::kThreads, 0, stream>>>(p, *shards);
  else
    attn_fwd_bf16_kernel<D, false><<<grid, C::kThreads, 0, stream>>>(p, ShardSrc{});
  return hipGetLastError();
}

template <class Tr, int D>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, const AttnDesc& d,
                  hipStream_t stream) {
  using C = FwdCfg<Tr, D>;
  FwdParams p;
  p.q = static_cast<const char*>(q);
  p.k = static_cast<const char*>(k);
  p.v = static_cast<const char*>(v);
  p.o = static_cast<char*>(o);
  p.lse = lse;
  p.cu = d.cu;
  p.ndocs = d.ndocs;
  p.N = static_cast<int>(d.N);
  p.hq = d.hq;
  p.hk = d.hk;
  p.G = d.hq / d.hk;
  p.Gw = std::gcd(p.G, C::kWaves);
  const int rows = C::RW * (C::kWaves / p.Gw);
  p.n_qtiles = static_cast<int>((d.N + rows - 1) / rows);
  p.scale_log2 = d.scale * kLog2e;
  p.causal = d.causal;
  dim3 grid(p.n_qtiles, d.hk * (p.G / p.Gw));
  attn_fwd_kernel<Tr, D><<<grid, C::kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_from_shards(const void* const* q_shards, const void* const* k_shards,
                                       const void* const* v_shards, int P, int64_t T, int Hq, int Hkv, int group,
                                       void* o, float* lse, const AttnDesc& d, hipStream_t stream) {
  ShardSrc sh{};
  for (int j = 0; j < P; ++j) {
    sh.q[j] = static_cast<const char*>(q_shards[j]);
    sh.k[j] = static_cast<const char*>(k_shards[j]);
    sh.v[j] = static_cast<const char*>(v_shards[j]);
  }
  sh.T = static_cast<int>(T);
  sh.q_row = Hq * d.D * 2;
  sh.kv_row = Hkv * d.D * 2;
  sh.q_head0 = group * d.hq;
  sh.kv_head0 = group * d.hk;
  return d.D == 128 ? launch_bf16<128>(nullptr, nullptr, nullptr, o, lse, d, stream, &sh)
                    : launch_bf16<64>(nullptr, nullptr, nullptr, o, lse, d, stream, &sh);
}

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           const AttnDesc& d, hipStream_t stream) {
  if (d.dt == ULY_BF16)
    return d.D == 128 ? launch_bf16<128>(q, k, v, o, lse, d, stream) : launch_bf16<64>(q, k, v, o, lse, d, stream);
  return d.D == 128 ? launch<TrF32, 128>(q, k, v, o, lse, d, stream)
                    : launch<TrF32, 64>(q, k, v, o, lse, d, stream);
}

}  // namespace uly
