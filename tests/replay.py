"""Replay a recorded parity case on the GPU against the oracle.

    python -m tests.replay test_reports/failures/<case>

Loads the bf16 inputs, workload and mode that tests/parity.py recorded when a
check failed, runs the C-ABI forward and backward on cuda:0 and the FP64
oracle, and prints, per output, the largest error over tolerance and the
integer mismatch counts (no assertion: the point is to look).
"""
import json
import sys

import numpy as np


def main(path):
    import torch

    import oracle
    from tests import parity

    d, w, mode = parity.load_case(path)
    print("case %s: %s mode %d" % (path, json.dumps({k: getattr(w, k) for k in ("B", "H", "N", "D", "causal")}), mode),
          flush=True)
    t = parity.to_dev(d, "cuda:0")
    f = parity.gpu_forward(t, w, mode)
    b = parity.gpu_backward(t, w, f, mode)
    torch.cuda.synchronize()
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=mode != 0, beta=w.beta)
    rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal)
    out = {
        "O": parity.ratio(parity.f64(f["o"]), ref["O"], ref["tol_O"]),
        "LSE": parity.ratio(parity.f64(f["lse"]), ref["lse"], ref["tol_lse"]),
        "dQ": parity.ratio(parity.f64(b["dq"]), rb["dQ"], rb["tol_dQ"]),
        "dK": parity.ratio(parity.f64(b["dk"]), rb["dK"], rb["tol_dK"]),
        "dV": parity.ratio(parity.f64(b["dv"]), rb["dV"], rb["tol_dV"]),
        "delta": parity.ratio(parity.f64(b["delta"]), rb["delta"], rb["tol_delta"]),
    }
    ok = ref["amb_tie"] == 0
    out["ties_mismatch"] = int(np.sum(f["ties"].cpu().numpy()[ok] != ref["ties"][ok]))
    okp = ok & (ref["amb_pbar"] == 0)
    out["pbar_one_mismatch"] = int(np.sum(f["pbar_one"].cpu().numpy()[okp] != ref["pbar_one"][okp]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
