"""The library keeps no state between calls: two problems launched at the same
time on two HIP streams (default priority) give, bit for bit, what each gives
alone on the current stream, in every mode, forward and backward."""
import numpy as np
import pytest

from numerics_safe_softmax_amd import inputs
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(nss, t, w, mode, stream):
    B, H, N, D = w.B, w.H, w.N, w.D
    dev = t["q"].device
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ints = [torch.empty((B, H, N), dtype=torch.int32, device=dev) for _ in range(3)]
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["q"]), torch.empty_like(t["q"])
    delta = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    kw = dict(scale=w.scale, causal=w.causal, stream=stream)
    nss.attn_fwd(t["q"], t["k"], t["v"], o, lse, ints[0], ints[1], ints[2], stabilise=mode, beta=w.beta, **kw)
    nss.attn_bwd(t["q"], t["k"], t["v"], o, t["dO"], lse, dq, dk, dv, delta, stabilise=mode, beta=w.beta, **kw)
    return {"o": o, "lse": lse, "ties": ints[0], "pbar_one": ints[1], "formed": ints[2], "dq": dq, "dk": dk,
            "dv": dv, "delta": delta}


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else (x.view(torch.int32) if x.dtype == torch.float32 else x)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_two_streams_match_one(mode):
    import numerics_safe_softmax_amd as nss
    wa = inputs.custom("streams", 2, 3, 700, 64, True, 41, tie_block=5, v_skew_dims=16, v_mu=-2.0, v_sigma=0.5,
                       do_mu=-0.5)
    wb = inputs.custom("streams", 1, 4, 513, 128, False, 42, v_skew_dims=32, v_mu=-2.0, v_sigma=0.5, do_mu=-0.5)
    ta = parity.to_dev(inputs.generate(wa), DEV)
    tb = parity.to_dev(inputs.generate(wb), DEV)
    cur = torch.cuda.current_stream()
    ra = _run(nss, ta, wa, mode, cur)
    rb = _run(nss, tb, wb, mode, cur)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    with torch.cuda.stream(sa):
        xa = _run(nss, ta, wa, mode, sa)
    with torch.cuda.stream(sb):
        xb = _run(nss, tb, wb, mode, sb)
    torch.cuda.synchronize()
    for ref, got, name in ((ra, xa, "a"), (rb, xb, "b")):
        for k in ref:
            assert torch.equal(_bits(ref[k]), _bits(got[k])), "%s: %s differs on a second stream" % (name, k)
