"""Pins for the FP64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: the pages'
rule table, exact rational brute force, closed forms of special cases, a
numpy float64 dense softmax attention, central finite differences of that
dense forward, and identities the gradient must satisfy.

Pages: itsolotime.com/archives/23922, sections "机制解释二" (P_bar, P, O and the
trigger) and "极简修复方案" (the shift rule and the claim that it leaves the
exact result unchanged and keeps max(P_bar) below 1); 91haoming.cn/news/
show-608006, section 三 (delta as a row-sum of an element-wise product).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from numerics_safe_softmax_amd import inputs
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(x):
    return inputs.to_bf16_bits(np.asarray(x, dtype=np.float64))


def vals(b):
    return inputs.bits_to_float(b).astype(np.float64)


def rand_problem(B, H, N, D, seed, scale_v=1.0):
    rng = np.random.default_rng(seed)
    q, k, v, g = (bits(rng.standard_normal((B, H, N, D)) * s) for s in (1, 1, scale_v, 1))
    return q, k, v, g


def dense_forward(qf, kf, vf, scale, causal):
    """numpy float64 softmax attention over [N, D] arrays (a second, independent path)."""
    S = scale * (qf @ kf.T)
    if causal:
        S = np.where(np.tril(np.ones_like(S, dtype=bool)), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    ell = E.sum(axis=1, keepdims=True)
    return (E / ell) @ vf, (m + np.log(ell))[:, 0]


# ------------------------------------------------------------------ rule table

def test_shift_rule_branch_table():
    g = json.load(open(os.path.join(GOLDEN, "shift_rule_table.json")))
    for c in g["cells"]:
        got = oracle.shift_rule(c["rm"], c["rs"], bool(c["stabilise"]), g["beta"])
        assert got == c["shift"], c


# ------------------------------------------------------------------ exact dots and ties

def test_exact_dot_against_fractions():
    rng = np.random.default_rng(3)
    for trial in range(300):
        d = int(rng.integers(1, 130))
        spread = int(rng.integers(0, 120))
        a = rng.standard_normal(d) * np.exp2(rng.integers(-spread, spread + 1, size=d))
        b = rng.standard_normal(d) * np.exp2(rng.integers(-spread, spread + 1, size=d))
        a = np.clip(a, -1e37, 1e37)
        b = np.clip(b, -1e37, 1e37)
        a[np.abs(a) < 1e-37] = 0.0
        b[np.abs(b) < 1e-37] = 0.0
        ab, bb = bits(a), bits(b)
        exact = brute.dot(ab, bb)
        val, fast = oracle.exact_dot(ab, bb)
        if fast:
            assert Fraction(val) == exact
        else:
            assert val == pytest.approx(float(exact), rel=1e-15, abs=1e-300)


def test_tie_counts_against_brute_force_small_integer_grids():
    rng = np.random.default_rng(5)
    for trial in range(40):
        N = int(rng.integers(1, 25))
        D = int(rng.choice([1, 2, 4, 8]))
        causal = bool(trial % 2)
        q = bits(rng.integers(-2, 3, size=(1, 1, N, D)) * 0.5)
        k = bits(rng.integers(-2, 3, size=(1, 1, N, D)) * 0.25)
        r = oracle.forward(q, k, scale=0.5, causal=causal, want=["ties", "rowmax", "amb_tie"])
        ref = brute.row_max_count(q[0, 0], k[0, 0], causal)
        for i, (m, c) in enumerate(ref):
            assert r["ties"][0, 0, i] == c
            assert r["rowmax"][0, 0, i] == float(Fraction(1, 2) * m)
            assert r["amb_tie"][0, 0, i] == 0          # small grids are exact in fp32 too


def test_tie_count_when_double_sums_are_not_exact():
    # q . k1 = 2^60 + 1 and q . k2 = 2^60: a double sum would call them tied
    D = 3
    q = bits([[[[2.0 ** 30, 1.0, 0.0]]]])
    q = np.repeat(q, 3, axis=2)
    k = bits([[[[2.0 ** 30, 1.0, 0.0], [2.0 ** 30, 0.0, 0.0], [0.0, 0.0, 1.0]]]])
    r = oracle.forward(q, k, scale=1.0, causal=False, want=["ties", "flags"])
    ref = brute.row_max_count(q[0, 0], k[0, 0], False)
    assert [int(t) for t in r["ties"][0, 0]] == [c for _, c in ref] == [1, 1, 1]
    assert np.all(r["flags"][0, 0] & 4)                    # the exact slow path decided
    # and the exact path still finds genuine ties: k2 == k1 bitwise
    k2 = k.copy()
    k2[0, 0, 1] = k2[0, 0, 0]
    r2 = oracle.forward(q, k2, scale=1.0, causal=False, want=["ties"])
    assert np.all(r2["ties"][0, 0] == 2)
    assert D == q.shape[-1]


def test_max_count_merge_over_partitions_equals_whole_row():
    # the (max, count) pair is a commutative monoid: any split of a row merges to the row's pair
    rng = np.random.default_rng(9)
    for trial in range(50):
        row = [Fraction(int(x)) for x in rng.integers(-3, 4, size=int(rng.integers(1, 40)))]
        whole = (max(row), sum(1 for x in row if x == max(row)))
        cuts = sorted(set(int(c) for c in rng.integers(1, len(row) + 1, size=4)))
        parts, start = [], 0
        for c in cuts + [len(row)]:
            if c > start:
                seg = row[start:c]
                parts.append((max(seg), sum(1 for x in seg if x == max(seg))))
                start = c
        rng.shuffle(parts)
        acc = parts[0]
        for p in parts[1:]:
            acc = brute.merge(acc, p)
        assert acc == whole


def test_ambiguity_flags():
    # different key vectors with the same exact dot, not exact in fp32: ambiguous
    q = bits([[[[1.0, 1.0 + 2 ** -7, 1.0 / 3, 3.0]]]])
    k_a = [0.7, 0.3, 0.9, 0.1]
    kb = bits([[[k_a, k_a[::-1], k_a]]])
    q3 = np.repeat(q, 3, axis=2)
    r = oracle.forward(q3, kb, scale=1.0, causal=False, want=["ties", "amb_tie"])
    raw = [brute.dot(q3[0, 0, 0], kb[0, 0, j]) for j in range(3)]
    exp_ties = sum(1 for x in raw if x == max(raw))
    assert r["ties"][0, 0, 0] == exp_ties
    # bitwise copies only: never ambiguous, even when fp32 sums round
    kc = bits([[[k_a, [0.0, 0.0, 0.0, -5.0], k_a]]])
    r2 = oracle.forward(q3, kc, scale=1.0, causal=False, want=["ties", "amb_tie"])
    assert r2["ties"][0, 0, 0] == 2 and r2["amb_tie"][0, 0, 0] == 0
    # a second key 2^-30 below the max: exact in double, merged by fp32 rounding: ambiguous
    qn = np.repeat(bits([[[[1.0, 2.0 ** -30, 0.0, 0.0]]]]), 3, axis=2)
    kn = bits([[[[1.0, 1.0, 0.0, 0.0], [1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, -5.0]]]])
    r3 = oracle.forward(qn, kn, scale=1.0, causal=False, want=["ties", "amb_tie"])
    assert r3["ties"][0, 0, 0] == 1 and r3["amb_tie"][0, 0, 0] == 1
    # the same gap at 2^-20 is exact in fp32: not ambiguous
    qe = np.repeat(bits([[[[1.0, 2.0 ** -20, 0.0, 0.0]]]]), 3, axis=2)
    r4 = oracle.forward(qe, kn, scale=1.0, causal=False, want=["ties", "amb_tie"])
    assert r4["ties"][0, 0, 0] == 1 and r4["amb_tie"][0, 0, 0] == 0


# ------------------------------------------------------------------ closed forms

def test_first_causal_row_sees_one_key():
    q, k, v, _ = rand_problem(2, 3, 17, 8, 21)
    r = oracle.forward(q, k, v, scale=0.3, causal=True, stabilise=True)
    assert np.array_equal(r["O"][:, :, 0, :], vals(v)[:, :, 0, :])
    s00 = 0.3 * np.sum(vals(q)[:, :, 0, :] * vals(k)[:, :, 0, :], axis=-1)
    assert np.allclose(r["lse"][:, :, 0], s00, rtol=0, atol=1e-14)
    assert np.all(r["ties"][:, :, 0] == 1)


def test_zero_queries_give_uniform_attention():
    _, k, v, _ = rand_problem(1, 2, 23, 8, 22)
    q = np.zeros_like(k)
    for causal in (True, False):
        r = oracle.forward(q, k, v, scale=0.125, causal=causal, stabilise=True)
        n = np.arange(1, 24) if causal else np.full(23, 23)
        assert np.allclose(r["lse"][0, 0], np.log(n), rtol=0, atol=1e-14)
        vf = vals(v)[0, 0]
        if causal:
            mean = np.cumsum(vf, axis=0) / n[:, None]
        else:
            mean = np.broadcast_to(vf.mean(axis=0), vf.shape)
        assert np.allclose(r["O"][0, 0], mean, rtol=1e-13, atol=1e-13)
        assert np.array_equal(r["ties"][0, 0], n)
        # rm == 0 with a repeated max: the rule's strict comparisons leave m* = 0 = rm
        assert np.all(r["shift"][0, 0] == 0.0)
        assert np.all(r["pbar_one"][0, 0][n > 1] == 1)
        assert np.all(r["flags"][0, 0][n > 1] & 1)


def test_two_visible_keys_is_a_logistic():
    q, k, v, _ = rand_problem(1, 1, 2, 16, 23)
    r = oracle.forward(q, k, v, scale=0.25, causal=True)
    qf, kf, vf = vals(q)[0, 0], vals(k)[0, 0], vals(v)[0, 0]
    s0, s1 = 0.25 * qf[1] @ kf[0], 0.25 * qf[1] @ kf[1]
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.allclose(r["O"][0, 0, 1], p0 * vf[0] + (1 - p0) * vf[1], rtol=1e-14, atol=1e-14)
    assert r["lse"][0, 0, 1] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s1 - s0))),
                                              abs=1e-14)


def test_constant_values_give_constant_output():
    q, k, _, _ = rand_problem(1, 2, 40, 16, 24)
    v = np.full_like(q, 0xC020)   # -2.5 everywhere
    r = oracle.forward(q, k, v, scale=0.25, causal=False, stabilise=True)
    assert np.allclose(r["O"], -2.5, rtol=1e-14, atol=0)
    assert np.allclose(r["O_stab"], -2.5, rtol=1e-14, atol=0)


def test_matches_dense_numpy_attention():
    for (N, D, causal, seed) in [(37, 16, True, 1), (64, 64, False, 2), (33, 128, True, 3)]:
        q, k, v, _ = rand_problem(2, 2, N, D, seed)
        sc = 1.0 / math.sqrt(D)
        r = oracle.forward(q, k, v, scale=sc, causal=causal)
        for b in range(2):
            for h in range(2):
                O, lse = dense_forward(vals(q)[b, h], vals(k)[b, h], vals(v)[b, h], sc, causal)
                assert np.allclose(r["O"][b, h], O, rtol=1e-12, atol=1e-12)
                assert np.allclose(r["lse"][b, h], lse, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ the fix's claims

@pytest.mark.parametrize("wname", ["tiny"])
def test_shift_invariance_and_invariant(wname):
    w = inputs.WORKLOADS[wname]
    d = inputs.generate(w)
    rs = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=True,
                        beta=w.beta)
    ru = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=False,
                        beta=w.beta)
    # exact arithmetic: the shift leaves the attention result unchanged
    err = np.linalg.norm(rs["O_stab"] - rs["O"]) / np.linalg.norm(rs["O"])
    assert err < 1e-13
    tie = rs["ties"] > 1
    assert tie.sum() >= 0.25 * w.N                          # the workload's duplicate-max rows
    rm = rs["rowmax"]
    # stabilised tie rows: max(P_bar) = exp((1 - beta) rm) or exp(rm), below 1
    want = np.where(rm > 0, np.exp((1 - w.beta) * rm), np.exp(rm))
    assert np.allclose(rs["pbar_max"][tie], want[tie], rtol=1e-14, atol=0)
    assert np.all(rs["pbar_max"][tie & (rm != 0)] < 1.0)
    assert np.all(rs["pbar_one"][tie & (rs["amb_pbar"] == 0) & (rm != 0)] == 0)
    # unstabilised rows, and stabilised rows without a repeat: max(P_bar) = 1 exactly
    assert np.all(ru["pbar_max"] == 1.0) and np.all(ru["pbar_one"] == 1)
    assert np.array_equal(rs["shift"][~tie], ru["shift"][~tie])
    assert np.all(rs["pbar_one"][~tie] == 1)
    # unstabilised tie rows form at least rs bf16 ones (each tied max gives exactly 1)
    assert np.all(ru["near_ones"][tie] >= ru["ties"][tie])


def test_sink_workload_has_four_maxima_everywhere():
    w = inputs.WORKLOADS["sink"]
    d = inputs.generate(w)
    rows = oracle.head_rows([0, 13, 47], w.N)
    r = oracle.forward(d["q"], d["k"], scale=w.scale, causal=False, stabilise=True, rows=rows,
                       want=["ties", "rowmax", "amb_tie", "pbar_max", "pbar_one"])
    t = r["ties"].reshape(-1)[rows]
    assert np.all(t == 4)
    assert np.all(r["rowmax"].reshape(-1)[rows] == 1.0)
    assert np.all(r["amb_tie"].reshape(-1)[rows] == 0)
    assert np.allclose(r["pbar_max"].reshape(-1)[rows], math.exp(-1.0), rtol=1e-15)
    assert np.all(r["pbar_one"].reshape(-1)[rows] == 0)


def test_gpt2_workload_tie_fraction():
    w = inputs.WORKLOADS["gpt2_small"]
    d = inputs.generate(w)
    rows = oracle.head_rows([0, 95], w.N)
    r = oracle.forward(d["q"], d["k"], scale=w.scale, causal=True, rows=rows, want=["ties"])
    t = r["ties"].reshape(-1)[rows]
    assert (t > 1).mean() >= 0.10


# ------------------------------------------------------------------ backward

def dense_loss(qf, kf, vf, gf, scale, causal):
    O, _ = dense_forward(qf, kf, vf, scale, causal)
    return float(np.sum(gf * O))


@pytest.mark.parametrize("causal", [True, False])
def test_backward_against_finite_differences(causal):
    N, D, sc = 6, 4, 0.7
    q, k, v, g = rand_problem(1, 1, N, D, 31 + causal)
    fw = oracle.forward(q, k, v, scale=sc, causal=causal)
    bw = oracle.backward(q, k, v, g, fw, scale=sc, causal=causal)
    base = [vals(x)[0, 0] for x in (q, k, v, g)]
    h = 1e-6
    for which, key in ((0, "dQ"), (1, "dK"), (2, "dV")):
        fd = np.zeros((N, D))
        for i in range(N):
            for c in range(D):
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][i, c] += h
                minus[which][i, c] -= h
                fd[i, c] = (dense_loss(*plus, sc, causal) - dense_loss(*minus, sc, causal)) / (2 * h)
        assert np.allclose(bw[key][0, 0], fd, rtol=1e-6, atol=1e-8), key


def test_gradient_identities():
    w = inputs.WORKLOADS["tiny"]
    d = inputs.generate(w)
    fw = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=True)
    bw = oracle.backward(d["q"], d["k"], d["v"], d["dO"], fw, scale=w.scale, causal=True)
    qf, kf, gf = vals(d["q"]), vals(d["k"]), vals(d["dO"])
    # adding one vector to every key shifts each score row by a constant
    assert np.allclose(bw["dK"].sum(axis=2), 0.0, atol=1e-12 * np.abs(bw["dK"]).sum())
    # each row of P sums to one
    assert np.allclose(bw["dV"].sum(axis=2), gf.sum(axis=2), rtol=1e-12, atol=1e-10)
    # both sides equal scale * dL/dscale
    assert np.sum(qf * bw["dQ"]) == pytest.approx(np.sum(kf * bw["dK"]), rel=1e-11)
    # delta is the row-sum of dO * O
    assert np.allclose(bw["delta"], np.sum(gf * fw["O"], axis=-1), rtol=1e-14, atol=1e-14)
    # tolerances are positive and finite everywhere
    for t in ("tol_delta", "tol_dQ", "tol_dK", "tol_dV"):
        assert np.all(np.isfinite(bw[t])) and np.all(bw[t] > 0)
    assert np.all(np.isfinite(fw["tol_O"])) and np.all(fw["tol_O"] > 0)


def test_zero_output_gradient_gives_zero_gradients():
    q, k, v, _ = rand_problem(1, 2, 20, 8, 41)
    g = np.zeros_like(q)
    fw = oracle.forward(q, k, v, scale=0.35, causal=True)
    bw = oracle.backward(q, k, v, g, fw, scale=0.35, causal=True)
    for f in ("delta", "dQ", "dK", "dV"):
        assert np.all(bw[f] == 0.0)


def test_backward_head_subset_matches_full():
    q, k, v, g = rand_problem(2, 2, 19, 8, 43)
    fw = oracle.forward(q, k, v, scale=0.35, causal=True)
    full = oracle.backward(q, k, v, g, fw, scale=0.35, causal=True)
    part = oracle.backward(q, k, v, g, fw, scale=0.35, causal=True, heads=[3])
    for f in ("dQ", "dK", "dV", "delta"):
        assert np.array_equal(part[f][1, 1], full[f][1, 1])
        assert np.all(np.isnan(part[f][0, 0]))


def test_generator_rounding_agrees_with_oracle_rne():
    rng = np.random.default_rng(51)
    x = rng.standard_normal(50000) * np.exp2(rng.integers(-100, 100, size=50000))
    assert np.array_equal(inputs.to_bf16_bits(x), oracle.bf16_from_double(x, "rne"))
