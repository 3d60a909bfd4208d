"""Signed-bias statistics of a bf16 kernel's outputs against the FP64 oracle.

TEST INFRASTRUCTURE (part of the oracle package): used by tests/ and by the
cpu_baseline leg of bench.py, on rows the oracle has computed.

The pages' claim (itsolotime.com/archives/23922, section "机制解释二"): with
repeated maxima, P_bar holds exact 1s, and where V is mostly negative the bf16
accumulation of P_bar V drifts negative, so O_lp sits below O_hp; with dO also
negative the error entering the backward through delta = rowsum(dO o O) is
positive.  The statistic: on rows whose maximum repeats (rs >= 2) and on the
negatively skewed V dimensions, the mean signed error of O in bf16 ulps of the
reference, and of delta in units of u * sum_c |dO_ic O_ic| (u = 2^-8), with a
row-clustered standard error (each row's mean is one sample) and z = mean/SEM.
Controls: rows without a repeat, and the other dimensions.

Pinned by tests/test_bias_stats.py: ulp_bf16 against the exhaustive bf16
grid, the statistics against constructed errors of known mean and
row-clustered spread, event_curve against a hand-built event array, and the
whole report against the row-sum reading on the sink workload.
"""
from __future__ import annotations

import math

import numpy as np

U_BF16 = 2.0 ** -8


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid at |x| (normal range)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7.0)


def _stats(per_row: np.ndarray) -> dict:
    per_row = per_row[np.isfinite(per_row)]
    n = int(per_row.size)
    if n == 0:
        return {"n_rows": 0, "mean": None, "sem": None, "z": None}
    mean = float(per_row.mean())
    sem = float(per_row.std(ddof=1) / math.sqrt(n)) if n > 1 else float("nan")
    z = mean / sem if sem and sem > 0 else float("nan")
    return {"n_rows": n, "mean": mean, "sem": sem, "z": z}


def o_bias(O_gpu, O_ref, rows_mask, dims, O_ref_rounded=None) -> dict:
    """Mean signed error of O (in bf16 ulps of the reference) over rows x dims.

    Against the exact reference the statistic also carries the bias that any
    bf16 output has once the reference's values cluster at a power of two
    (the grid spacing doubles there, so rounding errors measured in ulps of
    the reference are not symmetric); against the correctly rounded reference
    (``O_ref_rounded``, bf16 round-to-nearest-even of the exact value) that
    part cancels and what remains is the bias of the computation itself.
    """
    ref = O_ref if O_ref_rounded is None else O_ref_rounded
    e = (O_gpu[..., dims] - ref[..., dims]) / ulp_bf16(O_ref[..., dims])
    per_row = e.mean(axis=-1)[rows_mask]
    out = _stats(per_row)
    raw = (O_gpu[..., dims] - ref[..., dims]).mean(axis=-1)[rows_mask]
    out["mean_abs_units"] = float(raw.mean()) if raw.size else None
    return out


def delta_bias(delta_gpu, delta_ref, dO, O_ref, rows_mask) -> dict:
    """Mean signed error of delta in units of u * sum_c |dO_ic O_ic|."""
    scale = U_BF16 * np.sum(np.abs(dO * O_ref), axis=-1)
    e = (delta_gpu - delta_ref) / np.maximum(scale, 1e-300)
    out = _stats(e[rows_mask])
    raw = (delta_gpu - delta_ref)[rows_mask]
    out["mean_abs_units"] = float(raw.mean()) if raw.size else None
    return out


def mode_difference(a: dict, b: dict) -> float:
    """z of the difference of two means with independent standard errors."""
    if not a.get("n_rows") or not b.get("n_rows") or a["sem"] is None or b["sem"] is None:
        return float("nan")
    den = math.sqrt(a["sem"] ** 2 + b["sem"] ** 2)
    return (a["mean"] - b["mean"]) / den if den > 0 else float("nan")


def report(O_gpu, O_ref, delta_gpu, delta_ref, dO, ties, rows_mask, skew_dims: int,
           O_ref_rounded=None) -> dict:
    """Bias of O and delta on tie rows x skewed dims, with the two controls.

    With ``O_ref_rounded`` given, the O statistics are also reported against
    the correctly rounded reference, and delta against sum_c dO_ic * that
    rounded O (what an exactly rounded bf16 forward would hand the backward).
    """
    D = O_ref.shape[-1]
    skew = np.arange(skew_dims)
    rest = np.arange(skew_dims, D)
    tie = rows_mask & (ties >= 2)
    notie = rows_mask & (ties == 1)
    out = {
        "O_tie_rows_skewed_dims": o_bias(O_gpu, O_ref, tie, skew),
        "O_tie_rows_other_dims": o_bias(O_gpu, O_ref, tie, rest) if rest.size else None,
        "O_single_max_rows_skewed_dims": o_bias(O_gpu, O_ref, notie, skew),
        "delta_tie_rows": delta_bias(delta_gpu, delta_ref, dO, O_ref, tie),
        "delta_single_max_rows": delta_bias(delta_gpu, delta_ref, dO, O_ref, notie),
    }
    if O_ref_rounded is not None:
        d_round = np.sum(dO * O_ref_rounded, axis=-1)
        out["vs_rounded_reference"] = {
            "O_tie_rows_skewed_dims": o_bias(O_gpu, O_ref, tie, skew, O_ref_rounded),
            "O_single_max_rows_skewed_dims": o_bias(O_gpu, O_ref, notie, skew, O_ref_rounded),
            "delta_tie_rows": delta_bias(delta_gpu, d_round, dO, O_ref, tie),
            "delta_single_max_rows": delta_bias(delta_gpu, d_round, dO, O_ref, notie),
        }
    return out


def event_curve(O_emul, O_exact, events, rows_mask, skew_dims: int) -> dict:
    """Signed error of an emulated O against the exact one, in bf16 ulps of the
    exact value, on the skewed V dims, grouped by how many P_bar entries of
    the row equal 1 (the trigger of the pages' mechanism).  Per group: rows,
    mean, row-clustered SEM and z."""
    skew = np.arange(skew_dims)
    out = {}
    for lo, hi, name in ((0, 0, "0"), (1, 1, "1"), (2, 2, "2"), (3, 3, "3"), (4, 1 << 30, ">=4")):
        m = rows_mask & (events >= lo) & (events <= hi)
        if not m.any():
            continue
        e = (O_emul[..., skew] - O_exact[..., skew]) / ulp_bf16(O_exact[..., skew])
        st = _stats(e[m].mean(axis=-1))
        st["rows"] = st.pop("n_rows") if "n_rows" in st else int(m.sum())
        out[name] = st
    return out
