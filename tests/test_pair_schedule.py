"""Host: the placement of the causal dK/dV pass's paired key tiles.

`place_pairs` (numerics_safe_softmax_amd/csrc/pair_schedule.h) decides which
heavy + light pair of key tiles each paired workgroup of an XCD's round takes.
A wrong order would leave a key tile uncomputed (or computed twice) only on
the grids that take it, so the header is compiled here on its own with g++
and checked over every one-round grid shape: each pair exactly once, the
per-CU work at the bound the greedy rule promises on the GPT-2 small grid,
and the plain order kept where all pairs are equal and already head-aligned
(GPT-2 medium, long context)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "numerics_safe_softmax_amd", "csrc")

HARNESS = r"""
#include <cstdio>
#include "pair_schedule.h"
using nss::PairOrder;
using nss::place_pairs;

static int cost(int l, int hx, int nqt, int qpk) { return nqt - (l / hx) * qpk + 1; }

int main() {
  long checked = 0;
  for (int hx = 1; hx < 40; ++hx)
    for (int nkt = 1; nkt < 130; ++nkt) {
      const int nloc = hx * nkt;
      if (nloc <= 64 || nloc > 128) continue;
      const int single = 128 - nloc, np = (nloc - single) / 2;
      const int bqs[2] = {64, 32};
      for (int bq : bqs)
        for (int trim = 0; trim < 128; trim += 77) {
          const int N = nkt * 128 - trim;
          PairOrder o;
          for (int k = 0; k < 64; ++k) o.p[k] = 255;
          place_pairs(o, nloc, single, hx, (N + bq - 1) / bq, 128 / bq);
          bool seen[64] = {};
          for (int k = 0; k < np; ++k) {
            if (o.p[k] >= np || seen[o.p[k]]) {
              printf("BAD %d %d %d %d\n", hx, nkt, bq, N);
              return 1;
            }
            seen[o.p[k]] = true;
          }
          ++checked;
        }
    }
  printf("checked %ld\n", checked);
  // GPT-2 small: 12 heads per XCD, 8 key tiles, 16 query tiles of 64 rows
  {
    const int hx = 12, nloc = 96, single = 32, nqt = 16, qpk = 2;
    PairOrder o;
    place_pairs(o, nloc, single, hx, nqt, qpk);
    int worst = 0, aligned = 0;
    for (int c = 0; c < 32; ++c) {
      const int q = o.p[c];  // workgroup c + 32 holds pair slot c
      const int w = cost(c, hx, nqt, qpk) + cost(single + q, hx, nqt, qpk) + cost(nloc - 1 - q, hx, nqt, qpk);
      worst = w > worst ? w : worst;
      aligned += (c % hx) == ((single + q) % hx);
    }
    printf("small %d %d\n", worst, aligned);
  }
  // GPT-2 medium (16 heads per XCD) and long context (2 heads, 64 key tiles)
  const int shapes[2][4] = {{16, 128, 16, 2}, {2, 128, 256, 4}};
  for (const auto& sh : shapes) {
    PairOrder o;
    place_pairs(o, sh[1], 0, sh[0], sh[2], sh[3]);
    int plain = 1;
    for (int k = 0; k < 64; ++k) plain &= o.p[k] == k;
    printf("plain %d\n", plain);
  }
  return 0;
}
"""


def test_pair_placement(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    src = tmp_path / "pp.cpp"
    src.write_text(HARNESS)
    exe = tmp_path / "pp"
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    assert out[0] == "checked 1092"
    worst, aligned = map(int, out[1].split()[1:])
    # the per-CU bound: a 16-tile single plus the lightest pair (12), with
    # three prologues; 20 of the 32 CUs share a head between their workgroups
    assert worst == 31 and aligned == 20
    assert out[2] == "plain 1" and out[3] == "plain 1"
