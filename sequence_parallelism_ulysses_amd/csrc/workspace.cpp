// Workspace layout of the attention backward: host logic shared by the
// launchers (attn_bwd.hip, noalloc.hip) and the size query of the C ABI.
#include "internal.hpp"

namespace uly {

// Workgroups per dK/dV key block. Each key block's (query tile, head)
// iterations are dealt round-robin to this many workgroups, which then stream
// the same Q/dO tiles at about the same time (shared in L2) and balance the
// causal spread of work per key block; their fp32 partials are added in
// split order by a reduce kernel. Timed over 1, 2, 3, 4, 6 and 8 at 32k,
// 128k and 256k tokens (Llama-3.1-8B-shaped head group), 4 was fastest at
// every size (by 0.5-3 %).
int bwd_dkdv_splits(const AttnDesc& d) { return d.splits > 0 ? d.splits : 4; }

BwdWorkspace bwd_workspace_layout(const AttnDesc& d) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  BwdWorkspace w;
  const size_t row_bytes = up(size_t(4) * d.hq * d.N);
  w.delta = 0;
  w.lse2 = row_bytes;
  size_t at = 2 * row_bytes;
  if (d.dt == ULY_BF16) {
    // the maxima, then the fp16 operand copies
    w.absmax = at;
    at += up(size_t(kBwdMaxima) * 4);
    const size_t qb = up(size_t(2) * d.N * d.hq * d.D), kb = up(size_t(2) * d.N * d.hk * d.D);
    w.q16 = at;
    w.do16 = at + qb;
    w.k16 = at + 2 * qb;
    w.v16 = at + 2 * qb + kb;
    at += 2 * qb + 2 * kb;
  } else {
    w.absmax = w.q16 = w.do16 = w.k16 = w.v16 = 0;
  }
  w.part = at;
  const int s = bwd_dkdv_splits(d);
  const size_t part_bytes = s > 1 ? size_t(2) * s * d.N * d.hk * d.D * 4 : 0;
  w.total = w.part + part_bytes;
  return w;
}

size_t bwd_workspace_bytes(const AttnDesc& d) { return bwd_workspace_layout(d).total; }

}  // namespace uly
