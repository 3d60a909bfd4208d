"""Pins of the oracle's online count (oracle.online_ones): how many keys per
row get a P_bar that rounds to a bf16 1.0 when the duplicate-max rule of
itsolotime.com/archives/23922, section "极简修复方案", is applied to the
running (max, count) pair tile by tile.

* One tile spanning the row is the whole-row rule: the count equals the
  forward oracle's final-shift prediction (near_ones), in both modes.
* On integer score grids (scale 1, so scores are integers and every P_bar off
  the shift is at most e^-1) a key's P_bar is 1 exactly when its score equals
  the shift, and the count follows from integer comparisons alone: per tile,
  the keys equal to the running maximum, unless the rule has moved the shift
  off it (a repeated positive or negative maximum).
* Without the rule every occurrence of the row maximum is formed as a 1, so
  the online count is at least the tie count.
"""
import numpy as np
import pytest

import oracle
from numerics_safe_softmax_amd import inputs


def _brute(scores, causal, stabilise, tile):
    """Integer brute force of the online count for one head's [N, N] integer scores."""
    N = scores.shape[0]
    out = np.zeros(N, dtype=np.int64)
    for i in range(N):
        last = i if causal else N - 1
        m, c, n = None, 0, 0
        for t0 in range(0, last + 1, tile):
            keys = range(t0, min(t0 + tile, last + 1))
            tm = max(scores[i, j] for j in keys)
            tc = sum(1 for j in keys if scores[i, j] == tm)
            if m is None or tm > m:
                m, c = tm, tc
            elif tm == m:
                c += tc
            moved = stabilise and c > 1 and m != 0  # beta*m (m > 0) or 0 (m < 0): no score equals it
            if not moved:
                n += sum(1 for j in keys if scores[i, j] == m)
        out[i] = n
    return out


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("stabilise", [False, True])
@pytest.mark.parametrize("tile", [1, 3, 4, 7])
def test_integer_grid_brute_force(causal, stabilise, tile):
    rng = np.random.default_rng(100 + tile + 10 * causal + 20 * stabilise)
    B, H, N, D = 1, 3, 23, 8
    q = rng.integers(-2, 3, size=(B, H, N, D)).astype(np.float64)
    k = rng.integers(-2, 3, size=(B, H, N, D)).astype(np.float64)
    k[:, :, 5] = k[:, :, 2]          # repeated keys: repeated maxima in many rows
    k[:, :, 11] = k[:, :, 9]
    qb, kb = inputs.to_bf16_bits(q), inputs.to_bf16_bits(k)
    r = oracle.online_ones(qb, kb, scale=1.0, causal=causal, stabilise=stabilise, beta=2.0, tile=tile)
    assert np.all(r["amb"] == 0)
    for h in range(H):
        s = (q[0, h] @ k[0, h].T).astype(np.int64)
        np.testing.assert_array_equal(r["ones"][0, h], _brute(s, causal, stabilise, tile))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("stabilise", [False, True])
def test_one_tile_is_the_whole_row_rule(causal, stabilise):
    w = inputs.custom("online", 1, 2, 150, 64, causal, 31, tie_block=4 if causal else 0, v_skew_dims=16,
                      v_mu=-2.0, v_sigma=0.5, do_mu=-0.5)
    d = inputs.generate(w)
    r = oracle.online_ones(d["q"], d["k"], scale=w.scale, causal=causal, stabilise=stabilise, tile=w.N)
    f = oracle.forward(d["q"], d["k"], scale=w.scale, causal=causal, stabilise=stabilise,
                       want=["near_ones", "amb_near"])
    ok = (r["amb"] == 0) & (f["amb_near"] == 0)
    np.testing.assert_array_equal(r["ones"][ok], f["near_ones"][ok])


def test_plain_online_count_covers_every_tie():
    w = inputs.custom("online", 1, 2, 300, 64, True, 32, tie_block=3, v_skew_dims=16, v_mu=-2.0, v_sigma=0.5,
                      do_mu=-0.5)
    d = inputs.generate(w)
    r = oracle.online_ones(d["q"], d["k"], scale=w.scale, causal=True, stabilise=False, tile=64)
    f = oracle.forward(d["q"], d["k"], scale=w.scale, causal=True, want=["ties", "amb_tie"])
    ok = (r["amb"] == 0) & (f["amb_tie"] == 0)
    assert np.all(r["ones"][ok] >= f["ties"][ok])
    assert np.any(r["ones"][ok] > f["ties"][ok])   # transient maxima of earlier tiles form ones too
