"""GPU parity: the C-ABI HIP path against the FP64 oracle, element by element.

Small shapes span several 128-row workgroup tiles and 64-key tiles with a
ragged tail, in both modes, causal and not, for D = 64 and 128; the full-size
workloads are checked on sampled rows and heads in the launch configuration the
benchmark times.  Integers (duplicate counts, P_bar == 1 flags) must match
exactly off the rows the oracle marks as undecidable in fp32.
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

SMALL = [
    # (B, H, N, D, causal, seed, tie_block)
    (1, 2, 200, 64, True, 11, 5),
    (2, 1, 333, 64, False, 12, 0),
    (1, 2, 300, 128, True, 13, 6),
    (1, 1, 130, 128, False, 14, 0),
    (1, 3, 1000, 64, True, 15, 10),
    (1, 1, 65, 64, True, 16, 4),
    (1, 1, 1, 64, True, 17, 0),
    (1, 1, 1, 128, False, 18, 0),
    (1, 1, 64, 128, True, 19, 4),
    # B*H a multiple of 8: the XCD-grouped workgroup order, with ragged tails
    (1, 8, 1000, 64, True, 22, 10),
    (2, 4, 777, 128, False, 23, 0),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _small_workload(B, H, N, D, causal, seed, tie_block):
    return inputs.custom("parity", B, H, N, D, causal, seed, tie_block=tie_block,
                         v_skew_dims=D // 4, v_mu=-2.0, v_sigma=0.5, do_mu=-0.5)


MODES = [0, 1, 2]   # plain, online duplicate-max shift, exact final shift


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dH%dN%dD%d%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
def test_small_fwd_bwd_parity(case, mode):
    w = _small_workload(*case)
    _say("parity %s mode=%d" % (case, mode))
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    f = parity.gpu_forward(t, w, mode)
    b = parity.gpu_backward(t, w, f, mode)
    torch.cuda.synchronize()
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=mode != 0,
                         beta=w.beta)
    rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal)
    with parity.record_on_failure("parity_%s_m%d" % (case, mode), d, w, mode):
        fr = parity.check_forward(f, ref, label=str(case))
        br = parity.check_backward(b, rb, label=str(case))
        _say("  fwd %s bwd %s" % (fr, br))
        formed = f["formed_ones"].cpu().numpy()
        ok = ref["amb_tie"] == 0
        if mode == 0:
            # plain rows: each tied maximum is fed to P_bar V as an exact bf16 1.0
            assert np.all(formed[ok] >= ref["ties"][ok])
            assert np.all(f["pbar_one"].cpu().numpy() == 1)
        if mode == 2:
            # the exact-final-shift kernel forms exactly the bf16 ones the final shift predicts
            okn = ok & (ref["amb_near"] == 0)
            assert np.array_equal(formed[okn], ref["near_ones"][okn])


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dH%dN%dD%d%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
def test_online_formed_ones(case, mode):
    """The kernel's count of formed bf16 ones equals the oracle's online count
    (the rule applied to the running pair, tiles of the forward's width, in key order) on
    every row the oracle can decide: the transient exact 1 of a tie split
    across tiles included, bit for bit."""
    import numerics_safe_softmax_amd as nss
    w = _small_workload(*case)
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    f = parity.gpu_forward(t, w, mode)
    torch.cuda.synchronize()
    r = oracle.online_ones(d["q"], d["k"], scale=w.scale, causal=w.causal, stabilise=mode != 0, beta=w.beta,
                           tile=nss.fwd_key_tile(w.D))
    ok = r["amb"] == 0
    formed = f["formed_ones"].cpu().numpy()
    bad = int(np.sum(formed[ok] != r["ones"][ok]))
    _say("online formed ones %s mode=%d: %d rows decided, %d undecidable, %d mismatches" % (
        case, mode, int(ok.sum()), int((~ok).sum()), bad))
    with parity.record_on_failure("online_%s_m%d" % (case, mode), d, w, mode):
        assert bad == 0, "%d rows with a different formed-ones count" % bad


@pytest.mark.parametrize("case", SMALL[:5], ids=lambda c: "B%dH%dN%dD%d%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
def test_tiecount_parity(case):
    import numerics_safe_softmax_amd as nss
    w = _small_workload(*case)
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    r = nss.tiecount(t["q"], t["k"], scale=w.scale, causal=w.causal)
    f = parity.gpu_forward(t, w, 1)
    f2 = parity.gpu_forward(t, w, 2)
    torch.cuda.synchronize()
    ref = oracle.forward(d["q"], d["k"], scale=w.scale, causal=w.causal,
                         want=["ties", "amb_tie", "rowmax"])
    # both forward modes count the same duplicates as the detector
    assert np.array_equal(f["ties"].cpu().numpy(), f2["ties"].cpu().numpy())
    ok = ref["amb_tie"] == 0
    ties = r["ties"].cpu().numpy()
    assert np.array_equal(ties[ok], ref["ties"][ok])
    # the detector and the forward form the same fp32 scores: identical counts everywhere
    assert np.array_equal(ties, f["ties"].cpu().numpy())
    rm = r["rowmax"].cpu().numpy().astype(np.float64)
    assert np.allclose(rm, ref["rowmax"], rtol=2e-6, atol=1e-6)


# rows of 2 048 keys or more: the duplicate detector (attn_tiecount and the
# first pass of the exact-final-shift forward) streams 128-key tiles there
LONG_ROWS = [
    (1, 2, 2100, 64, True, 31, 20),
    (1, 2, 2111, 64, False, 32, 0),
    (1, 1, 3001, 128, True, 33, 25),
    (1, 1, 2049, 128, False, 34, 0),
]


@pytest.mark.parametrize("case", LONG_ROWS, ids=lambda c: "B%dH%dN%dD%d%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
def test_long_row_tiecount_and_exact_shift(case):
    import numerics_safe_softmax_amd as nss
    w = _small_workload(*case)
    _say("long-row detector %s" % (case,))
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    r = nss.tiecount(t["q"], t["k"], scale=w.scale, causal=w.causal)
    f1 = parity.gpu_forward(t, w, 1)
    f2 = parity.gpu_forward(t, w, 2)
    torch.cuda.synchronize()
    ties = r["ties"].cpu().numpy()
    # the 128-key detector and the 64-key forward form the same fp32 scores
    assert np.array_equal(ties, f1["ties"].cpu().numpy())
    assert np.array_equal(ties, f2["ties"].cpu().numpy())
    ref = oracle.forward(d["q"], d["k"], scale=w.scale, causal=w.causal, want=["ties", "amb_tie", "rowmax"])
    ok = ref["amb_tie"] == 0
    assert np.array_equal(ties[ok], ref["ties"][ok])
    assert np.allclose(r["rowmax"].cpu().numpy().astype(np.float64), ref["rowmax"], rtol=2e-6, atol=1e-6)
    rng = np.random.default_rng(case[5])
    rows = np.sort(rng.choice(w.B * w.H * w.N, 64, replace=False))
    rows = np.unique(np.concatenate([rows, [0, w.N - 1, w.B * w.H * w.N - 1]]))
    m = np.zeros(w.B * w.H * w.N, dtype=bool)
    m[rows] = True
    ref2 = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=True, beta=w.beta,
                          rows=rows, want=parity.FWD_WANT)
    with parity.record_on_failure("longrow_%s" % (case,), d, w, 2):
        parity.check_forward(f2, ref2, rows_mask=m.reshape(w.B, w.H, w.N), label="long rows %s" % (case,))


# Attention-sink rows: key 0 is every row's maximum from the first tile on and
# three exact copies of it sit further along, so most later tiles hold no
# value that reaches a row's running maximum (the forward skips their count,
# merge and rescale for the whole wave) while the tiles with a copy must add
# to the count.  N >= 2048 takes the 128-key detector tiles as well.
SINK = [
    (1, 2, 700, 64, False, 41),
    (1, 2, 600, 128, True, 42),
    (1, 1, 2100, 64, False, 43),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", SINK, ids=lambda c: "B%dH%dN%dD%d%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
def test_sink_rows_parity(case, mode):
    import numerics_safe_softmax_amd as nss
    B, H, N, D, causal, seed = case
    w = inputs.custom("sink_rows", B, H, N, D, causal, seed, sink=True, v_skew_dims=D // 2, v_mu=-2.0,
                      v_sigma=0.5, do_mu=-0.5)
    _say("sink rows %s mode=%d" % (case, mode))
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    f = parity.gpu_forward(t, w, mode)
    b = parity.gpu_backward(t, w, f, mode)
    r = nss.tiecount(t["q"], t["k"], scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=mode != 0,
                         beta=w.beta)
    rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal)
    with parity.record_on_failure("sink_%s_m%d" % (case, mode), d, w, mode):
        fr = parity.check_forward(f, ref, label=str(case))
        br = parity.check_backward(b, rb, label=str(case))
        _say("  fwd %s bwd %s" % (fr, br))
        ok = ref["amb_tie"] == 0
        ties = r["ties"].cpu().numpy()
        assert np.array_equal(ties[ok], ref["ties"][ok])
        assert np.array_equal(ties, f["ties"].cpu().numpy())
        # the workload does what it is for: repeated maxima on most rows
        assert np.mean(ref["ties"] > 1) > 0.5
        if mode:
            okp = (ref["ties"] > 1) & ok & (ref["amb_pbar"] == 0) & ((ref["flags"] & 1) == 0)
            assert np.all(f["pbar_one"].cpu().numpy()[okp] == 0)


def test_deterministic_reruns():
    w = _small_workload(2, 2, 700, 64, True, 21, 7)
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    outs = []
    for _ in range(2):
        f = parity.gpu_forward(t, w, 2)
        b = parity.gpu_backward(t, w, f, 2)
        torch.cuda.synchronize()
        outs.append({k: v.cpu().clone() for k, v in list(f.items()) + list(b.items())})
    for k in outs[0]:
        assert torch.equal(outs[0][k].view(torch.uint8) if outs[0][k].dtype == torch.bfloat16 else outs[0][k],
                           outs[1][k].view(torch.uint8) if outs[1][k].dtype == torch.bfloat16 else outs[1][k]), k


def test_empty_problems_are_no_ops():
    import numerics_safe_softmax_amd as nss
    for shape in [(0, 2, 16, 64), (1, 0, 16, 64), (1, 2, 0, 64)]:
        q = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        f = nss.forward(q, q.clone(), q.clone(), scale=0.125, causal=True, stabilise=True)
        b = nss.backward(q, q.clone(), q.clone(), f["o"], q.clone(), f["lse"], scale=0.125, causal=True)
        assert f["o"].numel() == 0 and b["dq"].numel() == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("wname,heads", [("tiny", [0]), ("gpt2_small", [0, 57, 95]),
                                          ("gpt2_medium", [5, 127]), ("sink", [0, 30]),
                                          ("long_context", [9])])
def test_workload_parity(wname, heads):
    """Full-size workloads in the launch configuration the benchmark times; the
    oracle computes every row of the sampled heads (forward and backward)."""
    w = inputs.WORKLOADS[wname]
    _say("workload %s heads %s" % (wname, heads))
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    rows = oracle.head_rows(heads, w.N)
    hm = np.zeros((w.B, w.H), dtype=bool)
    for x in heads:
        hm[x // w.H, x % w.H] = True
    rmask = np.repeat(hm[:, :, None], w.N, axis=2)
    for stabilise in MODES:
        f = parity.gpu_forward(t, w, stabilise)
        b = parity.gpu_backward(t, w, f, stabilise)
        torch.cuda.synchronize()
        ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal,
                             stabilise=stabilise != 0, beta=w.beta, rows=rows, want=parity.FWD_WANT)
        fr = parity.check_forward(f, ref, rows_mask=rmask, label="%s s=%d" % (wname, stabilise))
        rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal,
                             heads=heads)
        br = parity.check_backward(b, rb, heads=heads, label="%s s=%d" % (wname, stabilise))
        tie = rmask & (ref["ties"] > 1)
        _say("  s=%d fwd %s bwd %s tie rows %d" % (stabilise, fr, br, int(tie.sum())))
        if stabilise:
            ok = tie & (ref["amb_tie"] == 0) & (ref["amb_pbar"] == 0) & ((ref["flags"] & 1) == 0)
            assert np.all(f["pbar_one"].cpu().numpy()[ok] == 0)
        if stabilise == 2:
            okn = rmask & (ref["amb_tie"] == 0) & (ref["amb_near"] == 0)
            assert np.array_equal(f["formed_ones"].cpu().numpy()[okn], ref["near_ones"][okn])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", SMALL[:5] + SMALL[6:7], ids=lambda c: "B%dH%dN%dD%d%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n"))
def test_fp32_o_path(case, mode):
    """attn_fwd_o32 / attn_bwd_o32: the bf16 O is the nearest-even rounding of
    the fp32 O, the rest of the forward equals attn_fwd bit for bit, and delta
    taken from the fp32 O (and the gradients after it) match the oracle."""
    import numerics_safe_softmax_amd as nss
    w = _small_workload(*case)
    _say("fp32-O path %s mode=%d" % (case, mode))
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    f = nss.forward(t["q"], t["k"], t["v"], scale=w.scale, causal=w.causal, stabilise=mode, beta=w.beta, o32=True)
    f0 = parity.gpu_forward(t, w, mode)
    b = nss.backward(t["q"], t["k"], t["v"], f["o"], t["dO"], f["lse"], scale=w.scale, causal=w.causal,
                     stabilise=mode, beta=w.beta, o32=f["o32"])
    torch.cuda.synchronize()
    assert torch.equal(f["o32"].to(torch.bfloat16).view(torch.int16), f["o"].view(torch.int16))
    for key in ("o", "lse", "ties", "pbar_one", "formed_ones"):
        a, c = f[key], f0[key]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           c.view(torch.int16) if c.dtype == torch.bfloat16 else c), key
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, stabilise=mode != 0, beta=w.beta)
    rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=w.causal)
    r32 = parity.ratio(f["o32"].double().cpu().numpy(), ref["O"], ref["tol_O"])
    assert r32 <= 1.0
    br = parity.check_backward(b, rb, label="o32 " + str(case))
    _say("  O32 err/tol %.3f, bwd %s" % (r32, br))
