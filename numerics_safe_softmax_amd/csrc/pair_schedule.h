// pair_schedule.h -- host-side placement of the causal dK/dV pass's paired
// key tiles (plain C++: the kernel takes PairOrder by value, and the host
// tests compile this header on its own).
#pragma once

#include <stdint.h>

namespace nss {

// Which pair of key tiles each paired workgroup of an XCD's round takes (see
// launch_dkdv_t in attn_kernels.hip): slot s (workgroup single + s of the XCD) takes pair p[s],
// i.e. the XCD's key tiles single + p[s] and nloc - 1 - p[s].  Passed by value.
struct PairOrder {
  uint8_t p[64];
};

// Placement of the paired key tiles of one XCD's round of 64 workgroups (nloc
// key tiles, heaviest first, the XCD's key tile l being key tile l / hx of its
// head l % hx; nqt query tiles per head, qpk query tiles per key tile).  The
// dispatcher puts workgroups L and L + 256 on one CU, i.e. workgroups j and
// j + 32 of an XCD.  Each key tile costs its query tiles plus one for its
// prologue.  CUs are taken heaviest first (by the single key tile they hold)
// and each free pair slot gets the cheapest pair left; among equal ones, a
// pair whose first key tile has the head of the CU's other work (the two
// workgroups then stream the same Q and dO rows at about the same time, so
// they meet in the XCD's L2), and among those the slot's own pair.  Measured
// against the plain order (slot s takes pair s): gpt2_small dK/dV 38.6 ->
// 37.6 us (a balanced order without the head rule: 38.4 -> 38.3 us); the
// GPT-2 medium and long-context grids (equal pairs, already head-aligned)
// keep the plain order.
inline void place_pairs(PairOrder& ord, int nloc, int single, int hx, int nqt, int qpk) {
  auto cost = [&](int l) { return nqt - (l / hx) * qpk + 1; };
  const int npairs = (nloc - single) / 2;  // = 64 - single
  auto pcost = [&](int q) { return cost(single + q) + cost(nloc - 1 - q); };
  int fixed[32] = {}, fhead[32], nfree[32] = {}, freeslot[32][2], cu[32];
  bool used[64] = {};
  for (int c = 0; c < 32; ++c) fhead[c] = -1;
  for (int j = 0; j < 64; ++j) {
    const int c = j & 31;
    if (j < single) {
      fixed[c] += cost(j);
      if (fhead[c] < 0) fhead[c] = j % hx;
    } else {
      freeslot[c][nfree[c]++] = j - single;
    }
  }
  for (int c = 0; c < 32; ++c) cu[c] = c;
  for (int i = 1; i < 32; ++i)  // CUs by fixed work, heaviest first (stable)
    for (int k = i; k > 0 && fixed[cu[k]] > fixed[cu[k - 1]]; --k) {
      const int tmp = cu[k];
      cu[k] = cu[k - 1];
      cu[k - 1] = tmp;
    }
  for (int i = 0; i < 32; ++i) {
    const int c = cu[i];
    for (int f = 0; f < nfree[c]; ++f) {
      const int slot = freeslot[c][f];
      int mc = -1;
      for (int q = 0; q < npairs; ++q)
        if (!used[q] && (mc < 0 || pcost(q) < mc)) mc = pcost(q);
      int pick = -1, rank_best = 4;  // every candidate ranks 0..3
      for (int q = 0; q < npairs; ++q) {
        if (used[q] || pcost(q) != mc) continue;
        const bool aligned = fhead[c] < 0 || (single + q) % hx == fhead[c];
        const int rank = (aligned ? 0 : 2) + (q == slot ? 0 : 1);
        if (rank < rank_best) {
          rank_best = rank;
          pick = q;
        }
      }
      used[pick] = true;
      ord.p[slot] = (uint8_t)pick;
      if (fhead[c] < 0) fhead[c] = (single + pick) % hx;
    }
  }
}

}  // namespace nss
