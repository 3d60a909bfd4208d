"""Shared helpers of the GPU parity tests: run the C-ABI path on seeded inputs
and compare it element by element with the FP64 oracle."""
from __future__ import annotations

import contextlib
import dataclasses
import json
import os
import re

import numpy as np

import oracle
from numerics_safe_softmax_amd import inputs

# where the GPU tests write their reports and record failing cases
# (NSS_REPORT_DIR, default test_reports/ at the repository root)
REPORT_DIR = os.environ.get("NSS_REPORT_DIR",
                            os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "test_reports"))
FAIL_DIR = os.path.join(REPORT_DIR, "failures")

FWD_WANT = ["O", "tol_O", "lse", "tol_lse", "ties", "pbar_one", "amb_tie", "amb_pbar", "amb_near",
            "near_ones", "rowmax", "flags"]


def to_dev(d, dev):
    return {k: inputs.to_torch(v, dev) for k, v in d.items()}


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def gpu_forward(t, w, stabilise):
    import numerics_safe_softmax_amd as nss
    return nss.forward(t["q"], t["k"], t["v"], scale=w.scale, causal=w.causal, stabilise=stabilise,
                       beta=w.beta)


def gpu_backward(t, w, f, stabilise):
    import numerics_safe_softmax_amd as nss
    return nss.backward(t["q"], t["k"], t["v"], f["o"], t["dO"], f["lse"], scale=w.scale,
                        causal=w.causal, stabilise=stabilise, beta=w.beta)


def ratio(got, want, tol, mask=None):
    """Largest |got - want| / tol over the (optionally masked) elements; where
    the tolerance is 0 (e.g. dK = 0 exactly when Q = 0) only equality passes."""
    err = np.abs(got - want)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), np.where(err == 0, 0.0, np.inf))
    if mask is not None:
        r = r[mask]
    return float(np.max(r)) if r.size else 0.0


def check_forward(f, ref, rows_mask=None, label=""):
    """O and LSE within tolerance; ties and pbar_one bit-exact off the ambiguous rows."""
    m = np.ones(ref["lse"].shape, dtype=bool) if rows_mask is None else rows_mask
    O = f64(f["o"])
    lse = f64(f["lse"])
    rO = ratio(O, ref["O"], ref["tol_O"], m[..., None].repeat(O.shape[-1], axis=-1))
    rL = ratio(lse, ref["lse"], ref["tol_lse"], m)
    assert rO <= 1.0, "%s O max err/tol %.3f" % (label, rO)
    assert rL <= 1.0, "%s LSE max err/tol %.3f" % (label, rL)
    ok = m & (ref["amb_tie"] == 0)
    ties = f["ties"].cpu().numpy()
    bad = int(np.sum(ties[ok] != ref["ties"][ok]))
    assert bad == 0, "%s %d tie-count mismatches" % (label, bad)
    okp = ok & (ref["amb_pbar"] == 0)
    pone = f["pbar_one"].cpu().numpy()
    badp = int(np.sum(pone[okp] != ref["pbar_one"][okp]))
    assert badp == 0, "%s %d pbar_one mismatches" % (label, badp)
    return {"O": rO, "LSE": rL, "ambiguous_rows": int(np.sum(m & (ref["amb_tie"] != 0)))}


def check_backward(b, rb, heads=None, label=""):
    B, H, N, D = rb["dQ"].shape
    hm = np.zeros((B, H), dtype=bool)
    if heads is None:
        hm[:] = True
    else:
        for x in heads:
            hm[x // H, x % H] = True
    out = {}
    for name, key in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV")):
        got = f64(b[name])
        r = ratio(got[hm], rb[key][hm], rb["tol_" + key][hm])
        assert r <= 1.0, "%s %s max err/tol %.3f" % (label, key, r)
        out[key] = r
    r = ratio(f64(b["delta"])[hm], rb["delta"][hm], rb["tol_delta"][hm])
    assert r <= 1.0, "%s delta max err/tol %.3f" % (label, r)
    out["delta"] = r
    return out


def dump_case(path, d, w, mode, note=""):
    """Record one case: the bf16 bit patterns of every input (uint16 .npy), the
    workload that generated them and the mode, so that it can be replayed
    without regenerating (tests/replay.py)."""
    os.makedirs(path, exist_ok=True)
    for name, bits in d.items():
        np.save(os.path.join(path, name + ".npy"), np.ascontiguousarray(bits, dtype=np.uint16))
    meta = {"workload": dataclasses.asdict(w), "mode": int(mode), "note": note}
    with open(os.path.join(path, "case.json"), "w") as fh:
        json.dump(meta, fh, indent=1)
    return path


def load_case(path):
    """The inputs, workload and mode recorded by dump_case."""
    with open(os.path.join(path, "case.json")) as fh:
        meta = json.load(fh)
    w = inputs.Workload(**meta["workload"])
    d = {}
    for fn in sorted(os.listdir(path)):
        if fn.endswith(".npy"):
            d[fn[:-4]] = np.load(os.path.join(path, fn))
    return d, w, meta["mode"]


@contextlib.contextmanager
def record_on_failure(label, d, w, mode):
    """Run the checks in the block; if one fails, record the case's inputs under
    FAIL_DIR before the failure propagates."""
    try:
        yield
    except AssertionError as e:
        where = dump_case(os.path.join(FAIL_DIR, re.sub(r"[^A-Za-z0-9_.-]+", "_", label).strip("_")), d, w, mode,
                          note=str(e))
        print("recorded failing case in %s" % where, flush=True)
        raise

