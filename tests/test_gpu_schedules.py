"""GPU: the dispatch orders of resident causal grids.

When a causal grid is resident all at once, the forward and the dQ pass
reorder their workgroups (later dispatch bands reversed by groups of 8) and
the dQ and tie-count passes start the lighter query tiles later; where the
key tiles of an XCD exceed one round of the dK/dV pass (more than 64), its
workgroups take heavy + light pairs of key tiles.  These cases build grids
that take those paths (B*H a multiple of 8 with more than 256 workgroups,
partial bands, ragged N, d = 64 and 128, paired key tiles with and without an
odd count, and a grid whose B*H is not a multiple of 8), fill every output
with NaN first so that a tile the reordered grid skipped would show, and
compare sampled heads with the oracle (every head has query tiles in the
reversed bands)."""
import numpy as np
import pytest

import oracle
from numerics_safe_softmax_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
DEV = "cuda:0"

# (B, H, N, D, seed): causal grids of ceil(N/128) * B * H workgroups
CASES = [
    (1, 40, 1024, 64, 71),    # 320 workgroups: a partial second band
    (2, 24, 900, 64, 72),     # 384, ragged N
    (1, 96, 650, 64, 73),     # 576: three bands, the last partial; ragged
    (1, 48, 1000, 128, 74),   # 384 at d = 128 (resident up to 512)
    (3, 5, 1500, 64, 75),     # B*H = 15: the stagger without the band order
    (1, 24, 5400, 64, 76),    # dK/dV pairing: 129 key tiles per XCD (odd), one taken alone
    (1, 40, 1700, 128, 77),   # dK/dV pairing at d = 128: 70 key tiles per XCD
]


def _nan_like(t):
    out = torch.empty_like(t)
    if out.dtype == torch.bfloat16:
        out.view(torch.int16).fill_(0x7FC0)
    elif out.dtype == torch.float32:
        out.fill_(float("nan"))
    else:
        out.fill_(-12345)
    return out


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dN%dD%d" % c[:4])
def test_resident_causal_orders(case, mode):
    import numerics_safe_softmax_amd as nss
    B, H, N, D, seed = case
    w = inputs.custom("sched", B, H, N, D, True, seed, tie_block=9, v_skew_dims=D // 4, v_mu=-2.0, v_sigma=0.5,
                      do_mu=-0.5)
    print("schedules %s mode=%d" % (case, mode), flush=True)
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    q, k, v, g = t["q"], t["k"], t["v"], t["dO"]
    o = _nan_like(q)
    lse = _nan_like(torch.empty((B, H, N), dtype=torch.float32, device=DEV))
    ties = _nan_like(torch.empty((B, H, N), dtype=torch.int32, device=DEV))
    pone = _nan_like(ties)
    formed = _nan_like(ties)
    kw = dict(scale=w.scale, causal=True)
    nss.attn_fwd(q, k, v, o, lse, ties, pone, formed, stabilise=mode, beta=w.beta, **kw)
    dq, dk, dv = _nan_like(q), _nan_like(q), _nan_like(q)
    delta = _nan_like(lse)
    nss.attn_bwd_dq(q, k, v, o, g, lse, dq, delta, **kw)
    nss.attn_bwd_dkdv(q, k, v, g, lse, delta, dk, dv, **kw)
    torch.cuda.synchronize()
    # every element written (finite inputs give finite outputs)
    for name, x in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("delta", delta)):
        assert bool(torch.isfinite(x.float()).all()), "%s has unwritten or non-finite elements" % name
    for name, x in (("ties", ties), ("pbar_one", pone), ("formed_ones", formed)):
        assert int((x == -12345).sum()) == 0, "%s has unwritten elements" % name
    # sampled heads against the oracle: the first, the last and one between
    BH = B * H
    heads = sorted({0, BH - 1, min(BH - 1, (BH * 5) // 8)})
    rows = oracle.head_rows(heads, N)
    hm = np.zeros((B, H), dtype=bool)
    for x in heads:
        hm[x // H, x % H] = True
    rmask = np.repeat(hm[:, :, None], N, axis=2)
    f = {"o": o, "lse": lse, "ties": ties, "pbar_one": pone, "formed_ones": formed}
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=True, stabilise=True, beta=w.beta, rows=rows,
                         want=parity.FWD_WANT)
    with parity.record_on_failure("sched_%s_m%d" % (case, mode), d, w, mode):
        fr = parity.check_forward(f, ref, rows_mask=rmask, label="sched %s m%d" % (case, mode))
        rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=True, heads=heads)
        br = parity.check_backward({"dq": dq, "dk": dk, "dv": dv, "delta": delta}, rb, heads=heads,
                                   label="sched %s m%d" % (case, mode))
    print("  fwd %s bwd %s" % (fr, br), flush=True)
