// Key-stationary dK/dV kernel for bf16 inputs (see attn_bwd.hip for the
// backward as a whole). Kept in its own translation unit so the build can
// give it its own code-generation flags.
//
// A workgroup owns 128 keys of one kv head and walks the (q head, 64-query
// tile) iterations that can see them (split between p.splits workgroups).
// It runs 8 waves, two per SIMD: waves w and w+4 share the 32-key block
// w % 4 and take query rows [0, 32) and [32, 64) of every tile, so each wave
// holds 32x32 S/dP blocks instead of 64x32 and two waves fit a SIMD. Per
// wave and tile:
//   S  = Q K^T   (A: Q rows from LDS, B: this lane's K row in registers)
//   dP = dO V^T  (A: dO rows from LDS, B: V rows from an LDS tile of the
//                 workgroup's 128 keys, loaded once)
//   dV^T += dO^T P,  dK^T += Q^T dS  (A: ds_read_b64_tr_b16 of the Q/dO tiles)
// The S/dP accumulators hold one key column per lane, which is the B-operand
// layout of the last two products. At the end the two waves of a key block
// add their partial dK/dV through LDS.
#include "bwd_common.hpp"

namespace uly {
namespace {

template <int D>
struct KvBf {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kKeys = 128;  // four blocks of 32
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int RB = 2 * D;                   // bytes per LDS row
  static constexpr int TB = TileFmt<D>::kBytes;      // 64 rows
  static constexpr int VB = 2 * TB;                  // V rows of the 128 keys
  static constexpr int STAGE = 2 * TB + 2 * 64 * 4;  // Q, dO, lse2[64], delta[64]
  static constexpr int NSTAGE = 3;
  static constexpr int LDS = VB + NSTAGE * STAGE;
  static constexpr int LOADS = 2 * tile_loads<D, kThreads>() + 2;
  static constexpr int RED = 4 * 2 * DB * 16 * 64 * 4;  // pair reduction buffer
  static_assert(RED <= LDS, "reduction fits in the tile memory");
};

template <int D, bool kF32Out>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void dkdv_bf16_kernel(BwdParams p) {
  using C = KvBf<D>;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_char* vtile = (lds_char*)smem_raw;
  lds_char* ring = vtile + C::VB;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int kb = w & 3;   // key block
  const int qh = w >> 2;  // query rows [32 qh, 32 qh + 32) of each tile
  const int kvh = blockIdx.y;
  const int split = int(blockIdx.x) % p.splits;
  const int kv0 = (int(blockIdx.x) / p.splits) * C::kKeys;  // first tiles carry the most causal work
  const int kw0 = kv0 + 32 * kb;
  const bool active = kw0 < p.N;
  const int key = kw0 + l32;
  const int my_de = doc_of(p.cu, p.ndocs, p.N, min(key, p.N - 1)).end;
  const int w_de_first = doc_of(p.cu, p.ndocs, p.N, min(kw0, p.N - 1)).end;
  const int w_de_last = doc_of(p.cu, p.ndocs, p.N, min(kw0 + 31, p.N - 1)).end;
  const uint32_t kv_row = uint32_t(p.hk) * D * 2;
  const uint32_t q_row = uint32_t(p.hq) * D * 2;

  // V rows of the workgroup's keys -> LDS (two 64-row tiles), issued first.
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int r0 = kv0 + 64 * h2;
    const int rows = max(0, min(64, p.N - r0));
    const int64_t off = (int64_t(r0) * p.hk + kvh) * D * 2;
    issue_tile<D, C::kThreads>(make_rsrc(p.v + off, uint32_t(rows) * kv_row), kv_row, vtile + h2 * C::TB, tid);
  }

  // This lane's K row: B operand of S = Q K^T.
  bf16x8_t kf[C::KS];
  {
    const int64_t off = (int64_t(key) * p.hk + kvh) * D * 2 + half * 16;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      kf[ks] = key < p.N ? *reinterpret_cast<const bf16x8_t*>(p.k + off + ks * 32) : bf16x8_t{};
  }
  f32x16_t dkt[C::DB], dvt[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dkt[db] = dvt[db] = f32x16_t{};
  RowFragOffsets<D> ro;  // rows l%32 of a tile, k = 16 ks + 8 half
  TrFragOffsets<D> to;   // transposed reads over 16-row steps
  ro.init(lane);
  to.init(lane);

  // Queries that can see any of the 128 keys: [kv0, end of the last key's
  // document). The (q head, query tile) iterations over them, head-major, are
  // split evenly between p.splits workgroups; this one takes [it0, it1).
  const int q_end = doc_of(p.cu, p.ndocs, p.N, min(kv0 + C::kKeys - 1, p.N - 1)).end;
  const int qt0 = kv0 / BT;
  const int n_qt = (q_end - 1) / BT - qt0 + 1;
  const int n_it = n_qt * p.G;
  const int it0 = int(int64_t(n_it) * split / p.splits);
  const int it1 = int(int64_t(n_it) * (split + 1) / p.splits);

  auto issue = [&](int it) {
    lds_char* st = ring + ((it - it0) % C::NSTAGE) * C::STAGE;
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

  const int vrow_off = kb * 32 * C::RB;  // this wave's key block inside the V tile
  const int qrow_off = qh * 32 * C::RB;  // this wave's query rows inside a Q/dO tile

  for (int it = it0; it < it1; ++it) {
    if (it + 1 < it1) wait_vmcnt<C::LOADS>(); else wait_vmcnt<0>();
    __syncthreads();
    const int qs = (qt0 + it % n_qt) * BT;
    const int row0 = qs + 32 * qh;  // first query row of this wave
    const lds_char* qt = ring + ((it - it0) % C::NSTAGE) * C::STAGE;
    const lds_char* dt = qt + C::TB;
    typedef __attribute__((address_space(3))) const float lds_float;
    lds_float* fl = (lds_float*)(qt + 2 * C::TB);

    if (active && row0 + 31 >= kw0 && row0 < w_de_last) {
      const bool need_mask = (row0 < kw0 + 31) || (row0 + 32 > w_de_first);
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        s = mfma(frag_rows_at<D>(qt, ro.off[ks] + qrow_off), kf[ks], s);
        dp = mfma(frag_rows_at<D>(dt, ro.off[ks] + qrow_off), frag_rows_at<D>(vtile, ro.off[ks] + vrow_off), dp);
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qi = 32 * qh + 8 * r4 + 4 * half;  // first of 4 consecutive queries
        typedef __attribute__((address_space(3))) const f32x4_t lds_f32x4;
        const f32x4_t l4 = *(lds_f32x4*)(fl + qi);
        const f32x4_t d4 = *(lds_f32x4*)(fl + 64 + qi);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * r4 + j;
          float e = fast_exp2(fmaf(s[r], p.scale_log2, -l4[j]));
          if (need_mask) {
            const int q = qs + qi + j;
            if (q < key || q >= my_de) e = 0.f;
          }
          pv[r] = e;
          dsv[r] = e * (dp[r] - d4[j]);
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over this wave's 32 queries)
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2) {
        const bf16x8_t pf = make_frag<TrBF16>(&pv[st2 * 8]);
        const bf16x8_t sf = make_frag<TrBF16>(&dsv[st2 * 8]);
        const int k0 = (32 * qh + 16 * st2) * C::RB;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          dvt[db] = mfma(frag_tr_at(dt, to.off[0][db] + k0, to.off[1][db] + k0), pf, dvt[db]);
          dkt[db] = mfma(frag_tr_at(qt, to.off[0][db] + k0, to.off[1][db] + k0), sf, dkt[db]);
        }
      }
    }
    if (it + 2 < it1) issue(it + 2);
  }

  // The two waves of a key block add their halves through LDS.
  wait_vmcnt<0>();
  __syncthreads();
  typedef __attribute__((address_space(3))) float lds_fw;
  lds_fw* red = (lds_fw*)smem_raw;
  auto red_at = [&](int which, int db, int r) { return red + ((((kb * 2 + which) * C::DB + db) * 16 + r) * 64 + lane); };
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        *red_at(0, db, r) = dkt[db][r];
        *red_at(1, db, r) = dvt[db][r];
      }
  }
  __syncthreads();
  if (qh == 1) return;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkt[db][r] += *red_at(0, db, r);
      dvt[db][r] += *red_at(1, db, r);
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
