"""GPU parity sweep: seeded random small shapes and every tile-boundary length.

Each case runs the C-ABI forward and backward and compares them element by
element with the FP64 oracle (O, LSE, delta, dQ, dK, dV within tolerance;
duplicate counts and P_bar == 1 flags bit-exact off the rows the oracle marks
undecidable in fp32).  The boundary lengths straddle the 32-row wave blocks,
the 32-, 64- and 128-key / 64-query tiles and the 128-row workgroup tiles of
every kernel.
"""
import sys

import numpy as np
import pytest

import oracle
from numerics_safe_softmax_amd import inputs
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 5))
        N = int(rng.integers(1, 641))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        mode = int(rng.integers(0, 3))
        tie_block = int(rng.choice([0, 3, 5, 9])) if causal else 0
        out.append((B, H, N, D, causal, 1000 + i, tie_block, mode))
    return out


RANDOM = _random_cases(24, 2026)
BOUNDARY = [(1, 2, n, 64, True, 2100 + n, 4, 1) for n in (31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 192, 193,
                                                          255, 256, 257)]
BOUNDARY += [(1, 1, n, 128, False, 2400 + n, 0, 2) for n in (63, 65, 129, 255)]
# the d = 128 forward's 32-key tiles, online modes, causal and not
BOUNDARY += [(1, 2, n, 128, True, 2500 + n, 4, 1) for n in (31, 32, 33, 95, 96, 97, 161)]
BOUNDARY += [(1, 1, n, 128, False, 2600 + n, 0, 0) for n in (33, 97, 160)]


def _ident(c):
    return "B%dH%dN%dD%d%s_m%d" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n", c[7])


@pytest.mark.parametrize("case", RANDOM + BOUNDARY, ids=_ident)
def test_sweep_parity(case):
    B, H, N, D, causal, seed, tie_block, mode = case
    print("sweep %s" % (case,), flush=True)
    sys.stdout.flush()
    w = inputs.custom("sweep", B, H, N, D, causal, seed, tie_block=tie_block, v_skew_dims=D // 4, v_mu=-2.0,
                      v_sigma=0.5, do_mu=-0.5)
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    f = parity.gpu_forward(t, w, mode)
    b = parity.gpu_backward(t, w, f, mode)
    torch.cuda.synchronize()
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=mode != 0, beta=w.beta)
    rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal)
    with parity.record_on_failure("sweep_%s" % (case,), d, w, mode):
        parity.check_forward(f, ref, label=str(case))
        parity.check_backward(b, rb, label=str(case))


def _random_sink_cases(n, seed):
    """Seeded random shapes with attention-sink inputs (every row's maximum at
    key 0, exact copies of it further along) or injected ties, for the online
    modes' formed-ones count as well as the outputs."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 9))
        N = int(rng.integers(4, 900))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        mode = int(rng.integers(0, 2))
        sink = bool(rng.integers(0, 2))
        out.append((B, H, N, D, causal, 3000 + i, sink, mode))
    return out


@pytest.mark.parametrize("case", _random_sink_cases(48, 2027),
                         ids=lambda c: "B%dH%dN%dD%d%s_%s_m%d" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n",
                                                                 "sink" if c[6] else "ties", c[7]))
def test_sweep_online_counts(case):
    import numerics_safe_softmax_amd as nss
    B, H, N, D, causal, seed, sink, mode = case
    print("sweep online %s" % (case,), flush=True)
    sys.stdout.flush()
    kw = dict(sink=True) if sink else dict(tie_block=5 if causal else 0)
    w = inputs.custom("sweep_online", B, H, N, D, causal, seed, v_skew_dims=D // 4, v_mu=-2.0, v_sigma=0.5,
                      do_mu=-0.5, **kw)
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    f = parity.gpu_forward(t, w, mode)
    b = parity.gpu_backward(t, w, f, mode)
    torch.cuda.synchronize()
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=mode != 0, beta=w.beta)
    rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal)
    with parity.record_on_failure("sweep_online_%s" % (case,), d, w, mode):
        parity.check_forward(f, ref, label=str(case))
        parity.check_backward(b, rb, label=str(case))
        # the formed ones against the rule applied tile by tile at the forward's width
        on = oracle.online_ones(d["q"], d["k"], scale=w.scale, causal=w.causal, stabilise=mode == 1,
                                beta=w.beta, tile=nss.fwd_key_tile(D))
        ok = on["amb"] == 0
        assert np.array_equal(f["formed_ones"].cpu().numpy()[ok], on["ones"][ok])

