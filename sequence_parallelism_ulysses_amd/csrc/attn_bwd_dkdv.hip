// Key-stationary dK/dV kernel for bf16 inputs (see attn_bwd.hip for the
// backward as a whole).
//
// A workgroup owns 32 kP keys of one kv head (kP = 6 in use: 192 keys) and
// walks the (q head, 32-query tile) iterations that can see them (split
// between p.splits workgroups). Its 2 kP waves (three per SIMD) specialise:
//   producer wave kb (0 .. kP-1): S = Q K^T and dP = dO V^T for the 32-key
//       block kb (A: Q / dO rows from the staged tile, B: this lane's K and
//       V rows, held in registers), then P = exp(S - LSE) and
//       dS = P (dP - Delta) on the vector unit; P and dS go to LDS as
//       ready-made MFMA B fragments;
//   consumer wave kP + 2j + r: accumulates dV^T += dO^T P (r = 0) or
//       dK^T += Q^T dS (r = 1) for the 64 keys of blocks 2j and 2j + 1
//       (A: ds_read_b64_tr_b16 of the staged dO / Q tile, each read feeding
//       both blocks; B: the fragments), one tile behind the producers,
//       accumulating in registers.
// So while one wave of a SIMD is busy with exponentials another has matrix
// work, and no wave needs registers for both the K/V rows and the dK/dV
// accumulators. Each staged Q/dO tile serves all 32 kP keys, so the more
// keys a workgroup holds the fewer bytes it streams per product: six blocks
// (168 registers per wave, three waves per SIMD) stream a third fewer than
// four (256 registers, two waves per SIMD) and run the 128k workload's
// backward about 2.5 % faster. The first four consumer waves also issue the
// tile copies (a four-stage ring, one barrier per tile): a burst of copies
// stalls the issuing wave at the address unit, and right after the barrier
// the consumer has nothing urgent.
#include <type_traits>

#include "bwd_common.hpp"

namespace uly {
namespace {

template <int D, int kP>
struct KvWs {
  static constexpr int kProducerWaves = kP;  // one per 32-key block; as many consumers
  static constexpr int kWaves = 2 * kP;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kProducers = 64 * kP;  // waves 0 .. kP-1
  static constexpr int kKeys = 32 * kP;
  static constexpr int QT = 32;           // query rows per tile
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int RB = 2 * D;                 // bytes per LDS row
  static constexpr int TQ = QT * RB;               // one staged Q or dO tile
  static constexpr int STAGE = 2 * TQ + 2 * 256;   // Q, dO, lse2[64], delta[64] (first 32 used)
  static constexpr int NSTAGE = 4;
  static constexpr int RING = NSTAGE * STAGE;
  static constexpr int PDS_BLOCK = 4 * 64 * 16;    // P and dS fragments of one key block
  static constexpr int PDS = 2 * kP * PDS_BLOCK;   // two tiles in flight, kP key blocks
  static constexpr int LDS = RING + PDS;
  static constexpr int kCopiers = 256;              // the first four consumer waves
  static constexpr int LOADS = 2 * tile_loads<D, kCopiers, QT>() + 2;  // per copying lane per stage
};

template <int D, int kP, bool kF32Out>
__global__ __attribute__((amdgpu_flat_work_group_size(KvWs<D, kP>::kThreads, KvWs<D, kP>::kThreads),
                          amdgpu_waves_per_eu(kP / 2, kP / 2)))
void dkdv_bf16_kernel(BwdParams p) {
  using C = KvWs<D, kP>;
  static_assert(kP % 2 == 0 && kP >= 4, "consumers cover two key blocks each; four of them copy");
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS];
  lds_char* ring = (lds_char*)smem_raw;
  lds_char* pds = ring + C::RING;

  const int tid = threadIdx.x;
  const int w = uniform(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const bool producer = w < kP;
  const int kb = producer ? w : 0;
  const int kvh = blockIdx.y;
  const int split = int(blockIdx.x) % p.splits;
  // heaviest key blocks first: the first blocks of the sequence, or with a
  // few packed documents the blocks farthest from their document's end
  const int rank = int(blockIdx.x) / p.splits;
  const int kblock = (p.cu != nullptr && p.causal && p.ndocs < 64)
                         ? uniform(key_block_by_work_rank(p.cu, p.ndocs, p.N, C::kKeys, p.n_tiles, rank))
                         : rank;
  const int kv0 = kblock * C::kKeys;
  const int kw0 = kv0 + 32 * kb;
  const int key = kw0 + l32;
  const KeyBounds kbd(p, key, kw0);
  const int my_lo = kbd.my_lo, my_de = kbd.my_de;
  const int w_de_first = kbd.w_de_first, w_de_last = kbd.w_de_last;
  const uint32_t q_row = uint32_t(p.hq) * D * 2;
  const BwdScales sc = bwd_scales(p.absmax, p.scale);

  // Queries that can see any of the workgroup's keys: [first_query(kv0), end of
  // the last key's document). The (query tile, q head) iterations over them, tiles from the
  // last one down and heads innermost, are dealt round-robin to the p.splits
  // workgroups of the key block; this one runs its share as local
  // iterations [it0, it1). All workgroups thus walk the tiles in the same
  // order at about the same pace, so those resident at the same time stream
  // the same Q / dO tiles and share them in L2 instead of each fetching its
  // own from memory.
  const int q_end = doc_of(p.cu, p.ndocs, p.N, min(kv0 + C::kKeys - 1, p.N - 1)).end;
  const int qt0 = first_query(p, kv0) / C::QT;
  const int n_qt = (q_end - 1) / C::QT - qt0 + 1;
  const int n_it = n_qt * p.G;
  const int it0 = 0;
  const int it1 = max(0, (n_it - split + p.splits - 1) / p.splits);

  // Local iteration it is the (query tile, head) pair number split + it *
  // splits = qi * G + hi of the key block's walk. Each wave keeps cursors
  // (qi, hi) and advances them by additions, rather than dividing by G on
  // every iteration (a division is a long chain of scalar instructions on
  // each wave's critical path).
  struct Cursor {
    int qi, hi;
  };
  // (wave-uniform values, kept in scalar registers)
  const int step_q = uniform(p.splits / p.G), step_h = uniform(p.splits % p.G);
  const Cursor first{uniform(split / p.G), uniform(split % p.G)};
  auto advance = [&](Cursor& c) {
    const int h = c.hi + step_h;
    const bool wrap = h >= p.G;
    c.hi = uniform(wrap ? h - p.G : h);
    c.qi = uniform(c.qi + step_q + (wrap ? 1 : 0));
  };
  auto tile_q0 = [&](const Cursor& c) { return (qt0 + n_qt - 1 - c.qi) * C::QT; };
  auto tile_head = [&](const Cursor& c) { return kvh * p.G + c.hi; };
  auto stage = [&](int it) { return ring + ((it - it0) % C::NSTAGE) * C::STAGE; };
  // does a key block (first key kb0, seen from query lo_first on, its
  // documents ending by de_last) receive gradient from the tile at c?
  auto sees_block = [&](const Cursor& c, int kb0, int lo_first, int de_last) {
    const int qs = tile_q0(c);
    return kb0 < p.N && qs + C::QT - 1 >= lo_first && qs < de_last;
  };
  auto sees = [&](const Cursor& c) { return sees_block(c, kw0, kbd.w_lo_first, w_de_last); };
  // P (slots 0, 1) and dS (slots 2, 3) fragments of tile it for key block b
  auto pds_at = [&](int it, int b, int slot) {
    return pds + (((it & 1) * kP + b) * 4 + slot) * 1024 + lane * 16;
  };
  typedef __attribute__((address_space(3))) bf16x8_t lds_frag;

  if (producer) {
    // This lane's K and V rows: B operands of S = Q K^T and dP = dO V^T.
    bf16x8_t kf[C::KS], vf[C::KS];
    {
      const int64_t off = (int64_t(key) * p.hk + kvh) * D * 2 + half * 16;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        kf[ks] = key < p.N ? *reinterpret_cast<const bf16x8_t*>(p.k16 + off + ks * 32) : bf16x8_t{};
        vf[ks] = key < p.N ? *reinterpret_cast<const bf16x8_t*>(p.v16 + off + ks * 32) : bf16x8_t{};
      }
    }
    RowFragOffsets<D> ro;  // rows l%32 of a tile, k = 16 ks + 8 half
    ro.init(lane);

    Cursor cur = first;  // at iteration it
    for (int it = it0; it <= it1; ++it, advance(cur)) {
      __syncthreads();  // tile it has landed (the consumers waited for it)
      if (it < it1 && sees(cur)) {
        const int qs = tile_q0(cur);
        const lds_char* qt = stage(it);
        const lds_char* dt = qt + C::TQ;
        typedef __attribute__((address_space(3))) const float lds_float;
        lds_float* fl = (lds_float*)(qt + 2 * C::TQ);
        const bool need_mask = (qs < kbd.w_lo_last) || (qs + C::QT > w_de_first);
        // Operand reads run kAhead product steps ahead of the products
        // (all of them at once when the registers allow).
        constexpr int kAhead = kP > 4 ? 2 : C::KS;
        bf16x8_t qa[C::KS], da[C::KS];
#pragma unroll
        for (int ks = 0; ks < kAhead; ++ks) {
          qa[ks] = frag_rows_at<D>(qt, ro.off[ks]);
          da[ks] = frag_rows_at<D>(dt, ro.off[ks]);
        }
        // lane (key, half), slot r: query qs + 8 (r / 4) + 4 half + r % 4
        f32x4_t l4[4], d4[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          typedef __attribute__((address_space(3))) const f32x4_t lds_f32x4;
          l4[r4] = *(lds_f32x4*)(fl + 8 * r4 + 4 * half);
          d4[r4] = *(lds_f32x4*)(fl + 64 + 8 * r4 + 4 * half);
        }
        if constexpr (kAhead == C::KS) __builtin_amdgcn_sched_barrier(0);
        f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          if (ks + kAhead < C::KS) {
            qa[ks + kAhead] = frag_rows_at<D>(qt, ro.off[ks + kAhead]);
            da[ks + kAhead] = frag_rows_at<D>(dt, ro.off[ks + kAhead]);
          }
          s = mfma_f16(qa[ks], kf[ks], s);
          dp = mfma_f16(da[ks], vf[ks], dp);
        }
        auto probs = [&](auto masked) {
          float pv[16], dsv[16];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int qi = 8 * r4 + 4 * half;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 4 * r4 + j;
              // e = P * 2^15, dsv = dS * 2^eds (see BwdScales)
              float e = fast_exp2(fmaf(s[r], sc.c_s, -l4[r4][j]));
              if constexpr (decltype(masked)::value) {
                const int q = qs + qi + j;
                if (q < my_lo || q >= my_de) e = 0.f;
              }
              pv[r] = e;
              dsv[r] = e * fmaf(dp[r], sc.kd, -d4[r4][j]);
            }
          }
#pragma unroll
          for (int st2 = 0; st2 < 2; ++st2) {
            *(lds_frag*)pds_at(it, kb, st2) = make_frag_f16(&pv[st2 * 8]);
            *(lds_frag*)pds_at(it, kb, 2 + st2) = make_frag_f16(&dsv[st2 * 8]);
          }
        };
        // the element-wise mask only on tiles before some key's first query (the
        // diagonal tiles when causal) and tiles crossing a document end
        if (need_mask) probs(std::true_type{}); else probs(std::false_type{});
      } else if (it < it1) {
        // a consumer covers two key blocks and may still read this one's fragments
#pragma unroll
        for (int slot = 0; slot < 4; ++slot) *(lds_frag*)pds_at(it, kb, slot) = bf16x8_t{};
      }
    }
    return;
  }

  // consumer: dV^T += dO^T P (dk_role false) or dK^T += Q^T dS (true) over
  // the 32 queries of each tile, for key blocks cb and cb + 1
  const int cw = w - kP;
  const bool dk_role = cw & 1;
  const int cb = 2 * (cw >> 1);
  int cb_k0[2], cb_lo[2], cb_de[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    cb_k0[b] = kv0 + 32 * (cb + b);
    cb_lo[b] = uniform(first_query(p, cb_k0[b]));
    cb_de[b] = uniform(doc_of(p.cu, p.ndocs, p.N, min(cb_k0[b] + 31, p.N - 1)).end);
  }
  f32x16_t acc[2][C::DB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[b][db] = f32x16_t{};
  TrFragOffsets<D> to;  // transposed reads over 16-row steps
  to.init(lane);
  const int ctid = tid - C::kProducers;
  const bool copier = ctid < C::kCopiers;
  // The copies' source offsets follow the copy cursor by additions too:
  // elements (qs * hq + head) * D of Q / dO and head * N + qs of lse2 / delta,
  // in scalar registers.
  const int64_t e_q = int64_t(uniform(p.hq)) * D, e_n = uniform(p.N);
  const int64_t e_step = -int64_t(C::QT) * step_q * e_q + step_h * D, e_wrap = -int64_t(C::QT) * e_q - int64_t(p.G) * D;
  const int64_t f_step = -int64_t(C::QT) * step_q + step_h * e_n, f_wrap = -int64_t(C::QT) - int64_t(p.G) * e_n;
  Cursor c_issue = first;  // at the tile to copy next
  int64_t e_off = int64_t(tile_q0(first)) * e_q + int64_t(tile_head(first)) * D;
  int64_t f_off = int64_t(tile_head(first)) * e_n + tile_q0(first);
  auto advance_issue = [&]() {
    const bool wrap = c_issue.hi + step_h >= p.G;
    advance(c_issue);
    e_off += e_step + (wrap ? e_wrap : 0);
    f_off += f_step + (wrap ? f_wrap : 0);
  };
  auto issue = [&](int it) {
    lds_char* st = stage(it);
    const int qs = uniform(tile_q0(c_issue));
    const uint32_t rows = uint32_t(min(C::QT, p.N - qs));
    const char* qsrc = p.q16 + e_off * 2;
    const char* dsrc = p.do16 + e_off * 2;
    issue_tile<D, C::kCopiers, C::QT, true>(make_rsrc_uniform(qsrc, rows * q_row), q_row, st, ctid);
    issue_tile<D, C::kCopiers, C::QT, true>(make_rsrc_uniform(dsrc, rows * q_row), q_row, st + C::TQ, ctid);
    // lse2 and delta of the tile's rows (every copying wave copies the same values)
    dma_to_lds<4>(make_rsrc_uniform(p.lse2 + f_off, rows * 4), st + 2 * C::TQ, lane * 4);
    dma_to_lds<4>(make_rsrc_uniform(p.delta + f_off, rows * 4), st + 2 * C::TQ + 256, lane * 4);
  };
  if (copier && it0 < it1) issue(it0);
  advance_issue();
  if (copier && it0 + 1 < it1) issue(it0 + 1);
  advance_issue();
  Cursor c_jt = first;  // at the tile the consumers process next
  const int slot0 = dk_role ? 2 : 0;          // dS or P fragments
  const int src_off = dk_role ? 0 : C::TQ;    // Q or dO tile
  for (int it = it0; it <= it1; ++it) {
    // tile it must have landed before the barrier; it+1 may be in flight
    if (it + 1 < it1) wait_vmcnt<C::LOADS>(); else wait_vmcnt<0>();
    __syncthreads();
    // the stage of tile it-2 is free: its consumer pass ended last iteration
    if (copier && it + 2 < it1) issue(it + 2);
    advance_issue();
    const int jt = it - 1;  // the tile the producers finished last iteration
    const bool run = jt >= it0 && (sees_block(c_jt, cb_k0[0], cb_lo[0], cb_de[0]) ||
                                   sees_block(c_jt, cb_k0[1], cb_lo[1], cb_de[1]));
    if (jt >= it0) advance(c_jt);
    if (run) {
      const lds_char* src = stage(jt) + src_off;
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2) {
        const bf16x8_t f0 = *(const lds_frag*)pds_at(jt, cb, slot0 + st2);
        const bf16x8_t f1 = *(const lds_frag*)pds_at(jt, cb + 1, slot0 + st2);
        const int k0 = 16 * st2 * C::RB;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8_t a = frag_tr_at(src, to.off[0][db] + k0, to.off[1][db] + k0);
          acc[0][db] = mfma_f16(a, f0, acc[0][db]);
          acc[1][db] = mfma_f16(a, f1, acc[1][db]);
        }
      }
    }
  }

  // Epilogue: lane (key, half) of block b holds d = 32 db + acc_row(r, half).
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int bkey = cb_k0[b] + l32;
    if (bkey >= p.N) continue;
    if (p.splits > 1) {
      // fp32 partial sums, reduced in split order by dkdv_reduce_kernel
      float* part = dk_role ? p.part_dk : p.part_dv;
      const int64_t off = ((int64_t(split) * p.N + bkey) * p.hk + kvh) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = db * 32 + 8 * r4 + 4 * half;
          *reinterpret_cast<f32x4_t*>(part + off + d) =
              f32x4_t{acc[b][db][4 * r4], acc[b][db][4 * r4 + 1], acc[b][db][4 * r4 + 2], acc[b][db][4 * r4 + 3]};
        }
    } else {
      constexpr int OE = kF32Out ? 4 : 2;
      char* out = dk_role ? p.dk : p.dv;
      const float mul = dk_role ? sc.mul_dk : sc.mul_dv;
      const int64_t off = (int64_t(bkey) * p.hk + kvh) * D * OE;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = db * 32 + 8 * r4 + 4 * half;
          float x[4];
#pragma unroll
          for (int j2 = 0; j2 < 4; ++j2) x[j2] = acc[b][db][4 * r4 + j2] * mul;
          store4<kF32Out>(out + off + d * OE, x, p.accumulate);
        }
    }
  }
}

}  // namespace

// Producer waves (32 keys each) of the dK/dV kernel: six, so twelve waves,
// three per SIMD, and 192 keys per workgroup.
constexpr int kDkdvProducers = 6;

template <int D, bool kF32Out>
hipError_t launch_dkdv_bf16(BwdParams& p, int splits, int hk, hipStream_t stream) {
  using C = KvWs<D, kDkdvProducers>;
  p.n_tiles = (p.N + C::kKeys - 1) / C::kKeys;
  dkdv_bf16_kernel<D, kDkdvProducers, kF32Out><<<dim3(p.n_tiles * splits, hk), C::kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template hipError_t launch_dkdv_bf16<128, false>(BwdParams&, int, int, hipStream_t);
template hipError_t launch_dkdv_bf16<128, true>(BwdParams&, int, int, hipStream_t);
template hipError_t launch_dkdv_bf16<64, false>(BwdParams&, int, int, hipStream_t);
template hipError_t launch_dkdv_bf16<64, true>(BwdParams&, int, int, hipStream_t);

}  // namespace uly
