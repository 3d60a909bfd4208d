"""Pins of the signed-bias statistics (oracle/bias.py) on the CPU.

The statistic is the pages' claim turned into a number (itsolotime.com/
archives/23922, section 机制解释二: with repeated maxima and mostly negative V
the low-precision O drifts one way, and through delta = rowsum(dO o O),
91haoming.cn/news/show-608006 section 三, so does the backward).  Each piece
is checked against answers fixed independently of it: an exhaustive table of
the bf16 grid for ulp_bf16, constructed errors with known mean and
row-clustered standard error for o_bias / delta_bias / _stats, a hand-built
event array for event_curve, and, end to end, the normalisation reading of
O's row sum on the tie-heavy sink workload.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import bias
from numerics_safe_softmax_amd import inputs
from tests import kernel_model as km


def _bf16_value(codes):
    return (np.asarray(codes, dtype=np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_ulp_bf16_matches_the_exhaustive_grid():
    # every positive finite bf16 value x: the grid spacing above x
    codes = np.arange(0x0001, 0x7F7F, dtype=np.uint32)
    x, nxt = _bf16_value(codes), _bf16_value(codes + 1)
    spacing = nxt - x
    # the spacing holds on the whole interval [x, next): at x and a third of
    # the way to the next value, for either sign
    for pt in (x, x + spacing / 3.0):
        assert np.array_equal(bias.ulp_bf16(pt), spacing)
        assert np.array_equal(bias.ulp_bf16(-pt), spacing)
    # spot values: ulp(1) = 2^-7, ulp(1.99) = 2^-7, ulp(2) = 2^-6, ulp(-3) = 2^-6
    assert bias.ulp_bf16(np.array([1.0, 1.99, 2.0, -3.0])).tolist() == [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6]


def _grid(rows, dims, lo=1.125):
    """Reference values inside one binade [1, 2) (ulp 2^-7) and the ulp."""
    ref = np.full((rows, dims), lo)
    return ref, 2.0 ** -7


def test_constant_offset_gives_its_mean():
    ref, ulp = _grid(40, 8)
    got = ref + 0.25 * ulp
    mask = np.ones(40, dtype=bool)
    r = bias.o_bias(got, ref, mask, np.arange(8))
    assert r["n_rows"] == 40
    assert r["mean"] == pytest.approx(0.25, abs=1e-15)
    assert r["sem"] == pytest.approx(0.0, abs=1e-15)
    assert r["mean_abs_units"] == pytest.approx(0.25 * ulp, abs=1e-18)


def test_symmetric_noise_has_small_z_and_the_textbook_statistics():
    rng = np.random.default_rng(3)
    ref, ulp = _grid(500, 16)
    e = rng.standard_normal((500, 16))
    got = ref + e * ulp
    r = bias.o_bias(got, ref, np.ones(500, dtype=bool), np.arange(16))
    per_row = e.mean(axis=1)
    assert r["mean"] == pytest.approx(per_row.mean(), rel=1e-12)
    assert r["sem"] == pytest.approx(per_row.std(ddof=1) / math.sqrt(500), rel=1e-12)
    assert abs(r["z"]) < 3.0


def test_row_correlated_error_uses_the_row_clustered_sem():
    # each row carries one error shared by its dims (plus a little noise):
    # the rows are the independent samples, so the SEM is the spread of the
    # row means over sqrt(rows), sqrt(dims) times what treating every element
    # as a sample would give
    rng = np.random.default_rng(4)
    rows, dims = 300, 32
    ref, ulp = _grid(rows, dims)
    r_i = 0.5 + rng.standard_normal(rows)
    got = ref + (r_i[:, None] + 1e-3 * rng.standard_normal((rows, dims))) * ulp
    r = bias.o_bias(got, ref, np.ones(rows, dtype=bool), np.arange(dims))
    per_row = ((got - ref) / ulp).mean(axis=1)
    assert r["sem"] == pytest.approx(per_row.std(ddof=1) / math.sqrt(rows), rel=1e-12)
    naive = ((got - ref) / ulp).std(ddof=1) / math.sqrt(rows * dims)
    assert r["sem"] > 4.0 * naive
    assert r["z"] == pytest.approx(per_row.mean() / r["sem"], rel=1e-12)


def test_masks_and_dims_select_what_is_counted():
    ref, ulp = _grid(10, 6)
    got = ref.copy()
    got[:, :3] += ulp          # selected dims: +1 ulp
    got[:, 3:] -= 5 * ulp      # other dims: -5 ulp, must not count
    got[7:] += 100 * ulp       # rows outside the mask: must not count
    mask = np.zeros(10, dtype=bool)
    mask[:7] = True
    r = bias.o_bias(got, ref, mask, np.arange(3))
    assert r["n_rows"] == 7 and r["mean"] == pytest.approx(1.0, abs=1e-15)


def test_rounded_reference_removes_the_rounding_of_a_correct_result():
    # a bf16 result that is the correctly rounded exact value has zero error
    # against the rounded reference, whatever the exact values' distribution
    rng = np.random.default_rng(5)
    exact = -2.0 + 0.5 * rng.standard_normal((200, 16))
    rounded = inputs.bits_to_float(oracle.bf16_from_double(exact, "rne")).astype(np.float64)
    mask = np.ones(200, dtype=bool)
    r = bias.o_bias(rounded, exact, mask, np.arange(16), O_ref_rounded=rounded)
    assert r["mean"] == 0.0
    # against the exact value the same result shows the rounding itself
    r2 = bias.o_bias(rounded, exact, mask, np.arange(16))
    assert r2["mean"] != 0.0 and abs(r2["mean"]) < 0.5


def test_delta_bias_units():
    rng = np.random.default_rng(6)
    rows, D = 50, 8
    dO = rng.standard_normal((rows, D))
    O = rng.standard_normal((rows, D))
    d_ref = np.sum(dO * O, axis=1)
    unit = 2.0 ** -8 * np.sum(np.abs(dO * O), axis=1)
    r = bias.delta_bias(d_ref + 0.5 * unit, d_ref, dO, O, np.ones(rows, dtype=bool))
    assert r["mean"] == pytest.approx(0.5, rel=1e-12)
    assert r["sem"] == pytest.approx(0.0, abs=1e-12)


def test_mode_difference():
    a = {"n_rows": 5, "mean": 1.0, "sem": 0.3}
    b = {"n_rows": 5, "mean": 0.2, "sem": 0.4}
    assert bias.mode_difference(a, b) == pytest.approx(0.8 / 0.5, rel=1e-12)
    assert math.isnan(bias.mode_difference({"n_rows": 0, "mean": None, "sem": None}, b))


def test_event_curve_groups_rows_by_their_event_count():
    # rows with 0, 1, 2, 3 and 4+ exact ones; the error of group g is g ulps
    events = np.array([0, 0, 1, 1, 1, 2, 3, 3, 4, 7, 5])
    group = np.minimum(events, 4)
    rows, dims = events.size, 4
    exact, ulp = _grid(rows, dims)
    emul = exact + group[:, None] * ulp
    mask = np.ones(rows, dtype=bool)
    mask[10] = False                    # one row of group >= 4 left out
    out = bias.event_curve(emul, exact, events, mask, skew_dims=dims)
    assert set(out) == {"0", "1", "2", "3", ">=4"}
    want_rows = {"0": 2, "1": 3, "2": 1, "3": 2, ">=4": 2}
    for name, g in (("0", 0), ("1", 1), ("2", 2), ("3", 3), (">=4", 4)):
        assert out[name]["rows"] == want_rows[name]
        assert out[name]["mean"] == pytest.approx(g, abs=1e-15)
    # groups with no rows are absent
    assert set(bias.event_curve(emul, exact, np.zeros(rows, dtype=int), mask, dims)) == {"0"}


def test_report_splits_tie_and_single_max_rows():
    rows, D = 12, 8
    ref, ulp = _grid(rows, D)
    ties = np.array([1, 2, 3, 1, 1, 2, 1, 4, 1, 1, 2, 1])
    got = ref + np.where(ties[:, None] >= 2, 1.0, -1.0) * ulp
    dO = np.ones((rows, D))
    d_ref = np.sum(dO * ref, axis=1)
    rep = bias.report(got, ref, np.sum(dO * got, axis=1), d_ref, dO, ties, np.ones(rows, dtype=bool), skew_dims=4)
    assert rep["O_tie_rows_skewed_dims"]["n_rows"] == int((ties >= 2).sum())
    assert rep["O_tie_rows_skewed_dims"]["mean"] == pytest.approx(1.0)
    assert rep["O_single_max_rows_skewed_dims"]["mean"] == pytest.approx(-1.0)
    # delta error of a tie row: D ulps over u * sum |dO O| = u * D * 1.125
    assert rep["delta_tie_rows"]["mean"] == pytest.approx(ulp / (2.0 ** -8 * 1.125))


def test_sink_bias_follows_the_row_sum_reading():
    """End to end on four heads of the tie-heavy sink workload, plain and
    exact-shift modes: O divided by the fp32 sum of the unrounded P_bar while
    its numerator uses the bf16-rounded values is biased (|z| well above 3 on
    the skewed dims of the repeated-max rows); divided by the sum of the
    rounded values that P_bar V consumes (P = P_bar / rowsum(P_bar) with the
    BF16 P_bar, itsolotime.com/archives/23922 section 机制解释二), it is not."""
    w = inputs.WORKLOADS["sink"]
    d = inputs.generate(w)
    heads = [0, 17, 33, 46]
    rows = oracle.head_rows(heads, w.N)
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, rows=rows, want=["O", "ties"])
    O_round = inputs.bits_to_float(oracle.bf16_from_double(np.nan_to_num(ref["O"]), "rne")).astype(np.float64)
    zs = {}
    for mode in (0, 2):
        for reading in ("bf16", "fp32"):
            O = np.full(ref["O"].shape, np.nan)
            for g in heads:
                b, h = g // w.H, g % w.H
                f = km.forward_head(d["q"][b, h], d["k"][b, h], d["v"][b, h], w.scale, w.causal, mode, w.beta,
                                    row_sum=reading)
                O[b, h] = f["O"]
            mask = ~np.isnan(O[..., 0]) & (ref["ties"] >= 2)
            r = bias.o_bias(O, ref["O"], mask, np.arange(w.v_skew_dims), O_ref_rounded=O_round)
            zs[(mode, reading)] = r["z"]
    print("sink O bias z (mode, row sum):", {k: round(v, 1) for k, v in zs.items()})
    assert abs(zs[(0, "fp32")]) > 10 and abs(zs[(2, "fp32")]) > 10
    assert abs(zs[(0, "bf16")]) < 3 and abs(zs[(2, "bf16")]) < 3
