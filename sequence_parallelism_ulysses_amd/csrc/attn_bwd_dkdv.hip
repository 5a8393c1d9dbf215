// Key-stationary dK/dV kernel for bf16 inputs (see attn_bwd.hip for the
// backward as a whole). Kept in its own translation unit: with one wave per
// SIMD its schedule depends on compiler flags that the other kernels do not
// want (MFMA accumulators in VGPRs, an ILP-first scheduler), set per file by
// the build.
#include "bwd_common.hpp"

namespace uly {
namespace {

template <int D>
struct KvBf {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TB = TileFmt<D>::kBytes;
  static constexpr int STAGE = 2 * TB + 2 * 64 * 4;  // Q, dO, lse2[64], delta[64]
  static constexpr int NSTAGE = 3;
  static constexpr int LOADS = 2 * tile_loads<D, kThreads>() + 2;
};

template <int D, bool kF32Out>
__global__ __launch_bounds__(256, 1) void dkdv_bf16_kernel(BwdParams p) {
  using C = KvBf<D>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::NSTAGE * C::STAGE];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int kvh = blockIdx.y;
  const int split = int(blockIdx.x) % p.splits;
  const int kv0 = (int(blockIdx.x) / p.splits) * (32 * C::kWaves);  // first tiles carry the most causal work
  const int kw0 = kv0 + 32 * w;
  const bool active = kw0 < p.N;
  const int key = kw0 + l32;
  const int my_de = doc_of(p.cu, p.ndocs, p.N, min(key, p.N - 1)).end;
  const int w_de_first = doc_of(p.cu, p.ndocs, p.N, min(kw0, p.N - 1)).end;
  const int w_de_last = doc_of(p.cu, p.ndocs, p.N, min(kw0 + 31, p.N - 1)).end;

  // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T.
  bf16x8_t kf[C::KS], vf[C::KS];
  {
    const int64_t off = (int64_t(key) * p.hk + kvh) * D * 2 + half * 16;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      kf[ks] = key < p.N ? *reinterpret_cast<const bf16x8_t*>(p.k + off + ks * 32) : bf16x8_t{};
      vf[ks] = key < p.N ? *reinterpret_cast<const bf16x8_t*>(p.v + off + ks * 32) : bf16x8_t{};
    }
  }
  f32x16_t dkt[C::DB], dvt[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dkt[db] = dvt[db] = f32x16_t{};

  // Queries that can see any of the 128 keys: [kv0, end of the last key's
  // document). The (q head, query tile) iterations over them, head-major, are
  // split evenly between p.splits workgroups; this one takes [it0, it1).
  const int q_end = doc_of(p.cu, p.ndocs, p.N, min(kv0 + 32 * C::kWaves - 1, p.N - 1)).end;
  const int qt0 = kv0 / BT;
  const int n_qt = (q_end - 1) / BT - qt0 + 1;
  const int n_it = n_qt * p.G;
  const int it0 = int(int64_t(n_it) * split / p.splits);
  const int it1 = int(int64_t(n_it) * (split + 1) / p.splits);
  const uint32_t q_row = uint32_t(p.hq) * D * 2;

  auto issue = [&](int it) {
    lds_char* st = smem + ((it - it0) % C::NSTAGE) * C::STAGE;
    const int head = kvh * p.G + it / n_qt;
    const int qs = (qt0 + it % n_qt) * BT;
    const int rows = min(BT, p.N - qs);
    const int64_t off = (int64_t(qs) * p.hq + head) * D * 2;
    issue_tile<D, C::kThreads>(make_rsrc(p.q + off, uint32_t(rows) * q_row), q_row, st, tid);
    issue_tile<D, C::kThreads>(make_rsrc(p.dout + off, uint32_t(rows) * q_row), q_row, st + C::TB, tid);
    // 64 floats of lse2 and delta (every wave copies the same values)
    const int64_t foff = int64_t(head) * p.N + qs;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.lse2 + foff, uint32_t(rows) * 4),
                                             (__attribute__((address_space(3))) void*)(st + 2 * C::TB), 4, lane * 4, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(p.delta + foff, uint32_t(rows) * 4),
                                             (__attribute__((address_space(3))) void*)(st + 2 * C::TB + 256), 4, lane * 4,
                                             0, 0, 0);
  };
  if (it0 < it1) issue(it0);
  if (it0 + 1 < it1) issue(it0 + 1);

  for (int it = it0; it < it1; ++it) {
    if (it + 1 < it1) wait_vmcnt<C::LOADS>(); else wait_vmcnt<0>();
    __syncthreads();
    const int qs = (qt0 + it % n_qt) * BT;
    const lds_char* qt = smem + ((it - it0) % C::NSTAGE) * C::STAGE;
    const lds_char* dt = qt + C::TB;
    typedef __attribute__((address_space(3))) const float lds_float;
    lds_float* fl = (lds_float*)(qt + 2 * C::TB);

    if (active && qs + BT - 1 >= kw0 && qs < w_de_last) {
      const bool need_mask = (qs < kw0 + 31) || (qs + BT > w_de_first);
      f32x16_t s[2] = {f32x16_t{}, f32x16_t{}}, dp[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          s[qb] = mfma(frag_rows<D>(qt, qb * 32 + l32, ks * 16, half), kf[ks], s[qb]);
          dp[qb] = mfma(frag_rows<D>(dt, qb * 32 + l32, ks * 16, half), vf[ks], dp[qb]);
        }
      float pv[32], dsv[32];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int qi = qb * 32 + 8 * r4 + 4 * half;  // first of 4 consecutive queries
          typedef __attribute__((address_space(3))) const f32x4_t lds_f32x4;
          const f32x4_t l4 = *(lds_f32x4*)(fl + qi);
          const f32x4_t d4 = *(lds_f32x4*)(fl + 64 + qi);
          const float lv[4] = {l4[0], l4[1], l4[2], l4[3]};
          const float dv4[4] = {d4[0], d4[1], d4[2], d4[3]};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * r4 + j;
            float e = fast_exp2(fmaf(s[qb][r], p.scale_log2, -lv[j]));
            if (need_mask) {
              const int q = qs + qi + j;
              if (q < key || q >= my_de) e = 0.f;
            }
            pv[qb * 16 + r] = e;
            dsv[qb * 16 + r] = e * (dp[qb][r] - dv4[j]);
          }
        }
      // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over the tile's 64 queries)
#pragma unroll
      for (int st2 = 0; st2 < BT / 16; ++st2) {
        const bf16x8_t pf = make_frag<TrBF16>(&pv[st2 * 8]);
        const bf16x8_t sf = make_frag<TrBF16>(&dsv[st2 * 8]);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          dvt[db] = mfma(frag_cols_tr<D>(dt, st2 * 16, db * 32, lane), pf, dvt[db]);
          dkt[db] = mfma(frag_cols_tr<D>(qt, st2 * 16, db * 32, lane), sf, dkt[db]);
        }
      }
    }
    if (it + 2 < it1) issue(it + 2);
  }

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
        store4<kF32Out>(p.dk + off + d * OE, kx);
        store4<kF32Out>(p.dv + off + d * OE, vx);
      }
  }
}

}  // namespace

template <int D, bool kF32Out>
hipError_t launch_dkdv_bf16(const BwdParams& p, dim3 grid, hipStream_t stream) {
  dkdv_bf16_kernel<D, kF32Out><<<grid, KvBf<D>::kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template hipError_t launch_dkdv_bf16<128, false>(const BwdParams&, dim3, hipStream_t);
template hipError_t launch_dkdv_bf16<128, true>(const BwdParams&, dim3, hipStream_t);
template hipError_t launch_dkdv_bf16<64, false>(const BwdParams&, dim3, hipStream_t);
template hipError_t launch_dkdv_bf16<64, true>(const BwdParams&, dim3, hipStream_t);

}  // namespace uly
