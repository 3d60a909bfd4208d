"""Pins of the oracle's tolerance tensors from both sides (CPU).

The pages fix no tolerance; the oracle derives its element-wise bounds from
the arithmetic of a bf16 kernel with fp32 accumulation.  Two properties make
them mean something:

* wide enough: an independent model of that arithmetic (tests/kernel_model.py:
  bf16 operands, fp32 sums, P_bar rounded to bf16, O normalised by the sum of
  the rounded P_bar as in itsolotime.com/archives/23922 section 机制解释二,
  bf16 outputs) lands inside every tolerance with room to spare, in every
  mode, on the tiny workload and on one GPT-2-small head;
* narrow enough: plausible mistakes land outside -- one row of O scaled by
  (1 + 2^-6), the row's heaviest key dropped, LSE moved by 4 tolerances, dV
  from the unnormalised P_bar, delta missing one dimension, dQ missing one key,
  dK missing one query (where that term carries a tenth of the sum), and dS
  formed without -delta.
"""
import numpy as np
import pytest

import oracle
from numerics_safe_softmax_amd import inputs
from tests import kernel_model as km


def _ratio(got, want, tol):
    err = np.abs(np.asarray(got, dtype=np.float64) - want)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), np.where(err == 0, 0.0, np.inf))
    return float(np.max(r))


def _problem(wname, heads):
    w = inputs.WORKLOADS[wname]
    d = inputs.generate(w)
    return w, d, heads


CASES = [("tiny", [0]), ("gpt2_small", [5])]


@pytest.fixture(scope="module", params=CASES, ids=[c[0] for c in CASES])
def case(request):
    wname, heads = request.param
    w, d, heads = _problem(wname, heads)
    rows = oracle.head_rows(heads, w.N)
    out = {}
    for mode in (0, 1, 2):
        ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=mode != 0,
                             beta=w.beta, rows=rows, want=["O", "tol_O", "lse", "tol_lse", "ties", "rowmax"])
        rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal, heads=heads)
        out[mode] = (ref, rb)
    return w, d, heads, out


def _head(x, w, g):
    return x[g // w.H, g % w.H]


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_model_of_the_kernel_arithmetic_is_inside_every_tolerance(case, mode):
    w, d, heads, out = case
    ref, rb = out[mode]
    worst = {}
    for g in heads:
        hd = {n: _head(d[n], w, g) for n in ("q", "k", "v", "dO")}
        f = km.forward_head(hd["q"], hd["k"], hd["v"], w.scale, w.causal, mode, w.beta)
        b = km.backward_head(hd["q"], hd["k"], hd["v"], hd["dO"], f["O"], f["lse"], w.scale, w.causal)
        assert np.array_equal(f["ties"], _head(ref["ties"], w, g))
        pairs = {
            "O": (f["O"], _head(ref["O"], w, g), _head(ref["tol_O"], w, g)),
            "LSE": (f["lse"], _head(ref["lse"], w, g), _head(ref["tol_lse"], w, g)),
            "delta": (b["delta"], _head(rb["delta"], w, g), _head(rb["tol_delta"], w, g)),
            "dQ": (b["dQ"], _head(rb["dQ"], w, g), _head(rb["tol_dQ"], w, g)),
            "dK": (b["dK"], _head(rb["dK"], w, g), _head(rb["tol_dK"], w, g)),
            "dV": (b["dV"], _head(rb["dV"], w, g), _head(rb["tol_dV"], w, g)),
        }
        for name, (got, want, tol) in pairs.items():
            worst[name] = max(worst.get(name, 0.0), _ratio(got, want, tol))
    print("max err/tol of the arithmetic model:", {k: round(v, 3) for k, v in worst.items()})
    # inside with room to spare.  Every bound carries a factor 2 over its
    # first-order terms, so a correct bf16 result can reach 0.5 (O's own
    # rounding alone reaches it); 0.6 leaves the fp32 terms their share
    for name, r in worst.items():
        assert r <= 0.6, (name, r)


def _row_probs(d, w, g, i, mode_ref):
    """Exact P of row i of head g (float64, from the bf16 inputs)."""
    q = inputs.bits_to_float(_head(d["q"], w, g)).astype(np.float64)
    k = inputs.bits_to_float(_head(d["k"], w, g)).astype(np.float64)
    n = i + 1 if w.causal else w.N
    s = w.scale * (k[:n] @ q[i])
    p = np.exp(s - s.max())
    return p / p.sum()


def test_planted_forward_mistakes_exceed_the_tolerance(case):
    w, d, heads, out = case
    ref, _ = out[1]
    g = heads[0]
    O, tolO = _head(ref["O"], w, g), _head(ref["tol_O"], w, g)
    lse, tolL = _head(ref["lse"], w, g), _head(ref["tol_lse"], w, g)
    v = inputs.bits_to_float(_head(d["v"], w, g)).astype(np.float64)
    rng = np.random.default_rng(7)
    rows = rng.choice(np.arange(16, w.N), size=8, replace=False)
    for i in rows:
        # one row of O scaled by (1 + 2^-6)
        assert _ratio(O[i] * (1 + 2.0 ** -6), O[i], tolO[i]) > 1.0, ("O x (1 + 2^-6)", i)
        # the row's heaviest key dropped (the rest renormalised)
        p = _row_probs(d, w, g, i, ref)
        j = int(np.argmax(p))
        keep = np.ones(p.size, dtype=bool)
        keep[j] = False
        O_drop = (p[keep] @ v[:p.size][keep]) / p[keep].sum()
        assert _ratio(O_drop, O[i], tolO[i]) > 1.0, ("key dropped", i)
    # LSE moved by four tolerances
    assert _ratio(lse + 4 * tolL, lse, tolL) == pytest.approx(4.0, rel=1e-9)


def test_planted_backward_mistakes_exceed_the_tolerance(case):
    w, d, heads, out = case
    ref, rb = out[1]
    g = heads[0]
    q = inputs.bits_to_float(_head(d["q"], w, g)).astype(np.float64)
    k = inputs.bits_to_float(_head(d["k"], w, g)).astype(np.float64)
    v = inputs.bits_to_float(_head(d["v"], w, g)).astype(np.float64)
    dO = inputs.bits_to_float(_head(d["dO"], w, g)).astype(np.float64)
    O, lse = _head(ref["O"], w, g), _head(ref["lse"], w, g)
    delta, tol_d = _head(rb["delta"], w, g), _head(rb["tol_delta"], w, g)
    dQ, dK, dV = (_head(rb[n], w, g) for n in ("dQ", "dK", "dV"))
    tQ, tK, tV = (_head(rb["tol_" + n], w, g) for n in ("dQ", "dK", "dV"))
    N = w.N
    S = w.scale * (q @ k.T)
    vis = np.tril(np.ones((N, N), dtype=bool)) if w.causal else np.ones((N, N), dtype=bool)
    S = np.where(vis, S, -np.inf)
    P = np.exp(S - lse[:, None])
    dP = dO @ v.T
    dS = P * (dP - delta[:, None])
    rows = np.arange(1, N)            # row 0 of a causal head sees one key: dS = 0 there

    def caught(got, want, tol):       # per row: some element outside its tolerance
        return np.max(np.abs(got - want) / tol, axis=-1) > 1.0

    # delta missing its largest term: every row
    c = np.argmax(np.abs(dO * O), axis=1)
    assert np.all(np.abs(dO[rows, c[rows]] * O[rows, c[rows]]) > tol_d[rows])
    # dS formed without -delta (dS = P dP): every key row of dK; in dQ_i the
    # mistake is -scale delta_i sum_j P_ij k_j, which vanishes where the
    # attention-weighted mean key is near 0 in every dimension: nearly every row
    dS_nod = P * dP
    assert np.all(caught(w.scale * dS_nod.T @ q, dK, tK)[:N - 1])
    nod_q = caught(w.scale * dS_nod @ k, dQ, tQ)[rows]
    assert nod_q.mean() >= 0.9, nod_q.mean()
    # dQ missing the key with the largest |dS|, dK missing the query with the
    # largest |dS|: caught wherever that entry carries a tenth of the row's
    # (key's) sum of |dS|.  A lighter single term can hide in the bound: each
    # row's delta error enters dK through every query term by magnitude.
    jq = np.argmax(np.abs(dS), axis=1)
    drop_q = dQ - w.scale * dS[np.arange(N), jq][:, None] * k[jq]
    heavy_q = np.abs(dS).max(axis=1) >= 0.1 * np.abs(dS).sum(axis=1)
    ok_q = caught(drop_q, dQ, tQ)
    # (rows with at least 8 visible keys: with two keys the entries of dS are
    # equal and opposite, and the bound of the row's delta error dominates)
    assert np.all(ok_q[heavy_q & (np.arange(N) >= 7)])
    ik = np.argmax(np.abs(dS), axis=0)
    drop_k = dK - w.scale * dS[ik, np.arange(N)][:, None] * q[ik]
    heavy_k = np.abs(dS).max(axis=0) >= 0.1 * np.abs(dS).sum(axis=0)
    ok_k = caught(drop_k, dK, tK)
    assert np.all(ok_k[heavy_k & (np.arange(N) < N - 1)])
    print("rows caught: dQ without -delta %.3f; single term dropped: dQ %.3f, dK %.3f"
          % (nod_q.mean(), ok_q[1:].mean(), ok_k[:N - 1].mean()))
    # dV from the unnormalised P_bar = exp(S - rm) instead of exp(S - LSE):
    # every key row that some query with more than one visible key sees
    Pbar = np.exp(S - S.max(axis=1, keepdims=True))
    assert np.mean(caught(Pbar.T @ dO, dV, tV)) > 0.99
