"""Degenerate and extreme cases of the method on the GPU, against the oracle.

* Q = 0: every score is 0, so every visible key ties at rm = 0; the rule's
  strict comparisons fall through to m = rm (itsolotime.com/archives/23922,
  section 极简修复方案), P_bar = 1 everywhere and pbar_one = 1 even when
  stabilising; O is the running mean of V and LSE = ln(visible keys).
* A repeated maximum that is negative: the rule shifts by 0, so the largest
  P_bar is exp(rm) < 1 and pbar_one = 0.
* A long sequence (N = 32768, d = 128): forward parity on sampled rows, in the
  launch configuration of any other call (64-bit offsets, many KV tiles).
* Repeated maxima placed at chosen key positions: in one 32-lane half, across
  the two halves of a 32-key block, across the two blocks of a 64-key tile,
  across tiles, three-way, and a single maximum on the ragged last key; the
  duplicate count must be exact whichever lanes and tiles hold the copies.
* Tensors beyond 2^31 elements (4 GiB of bf16): seven seeded heads, checked
  against the oracle, are replicated over B*H heads (head g holds head g mod 7,
  so a 2^31-element wrap would land on a different head); forward and backward
  on the big problem must reproduce the seven heads' outputs bit for bit in
  every one of its heads.
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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(x):
    return inputs.to_bf16_bits(np.asarray(x, dtype=np.float64))


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("D", [64, 128])
def test_zero_queries_tie_at_zero(mode, D):
    import numerics_safe_softmax_amd as nss
    rng = np.random.default_rng(40 + D)
    B, H, N = 1, 2, 300
    q = _bits(np.zeros((B, H, N, D)))
    k = _bits(rng.standard_normal((B, H, N, D)))
    v = _bits(rng.standard_normal((B, H, N, D)))
    dO = _bits(rng.standard_normal((B, H, N, D)))
    t = {n: inputs.to_torch(x, DEV) for n, x in (("q", q), ("k", k), ("v", v), ("dO", dO))}
    f = nss.forward(t["q"], t["k"], t["v"], scale=D ** -0.5, causal=True, stabilise=mode, beta=2.0)
    b = nss.backward(t["q"], t["k"], t["v"], f["o"], t["dO"], f["lse"], scale=D ** -0.5, causal=True)
    torch.cuda.synchronize()
    ref = oracle.forward(q, k, v, scale=D ** -0.5, causal=True, stabilise=mode != 0, beta=2.0)
    rb = oracle.backward(q, k, v, dO, ref, scale=D ** -0.5, causal=True)
    fr = parity.check_forward(f, ref, label="Q=0 D%d mode %d" % (D, mode))
    br = parity.check_backward(b, rb, label="Q=0")
    visible = np.arange(1, N + 1)
    assert np.array_equal(f["ties"].cpu().numpy()[0, 0], visible)
    assert np.all(f["pbar_one"].cpu().numpy() == 1)          # rm == 0: the rule does not fire
    assert np.all(ref["flags"][..., 1:] & 1)                 # the oracle flags every tied row (R4)
    assert not np.any(ref["flags"][..., 0] & 1)              # row 0 sees one key: no tie
    lse = f["lse"].cpu().numpy()[0, 0].astype(np.float64)
    assert np.allclose(lse, np.log(visible), rtol=0, atol=1e-5)
    _say("  Q=0 D%d mode %d fwd %s bwd %s" % (D, mode, fr, br))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_negative_repeated_maximum(mode):
    """Keys point away from the queries (all scores negative); the argmax key
    of each row is duplicated at an earlier position."""
    import numerics_safe_softmax_amd as nss
    rng = np.random.default_rng(77)
    B, H, N, D = 1, 1, 256, 64
    base = rng.standard_normal(D)
    qf = base + 0.1 * rng.standard_normal((B, H, N, D))
    kf = -base - 0.3 * rng.standard_normal((B, H, N, D))
    q, k = _bits(qf), _bits(kf)
    qd, kd = inputs.bits_to_float(q).astype(np.float64), inputs.bits_to_float(k).astype(np.float64)
    for i in range(8, N, 7):                     # copy row i's best key to an earlier slot
        s = kd[0, 0, :i + 1] @ qd[0, 0, i]
        j = int(np.argmax(s))
        slot = (j + 3) % i if (j + 3) % i != j else (j + 1) % i
        k[0, 0, slot] = k[0, 0, j]
        kd[0, 0, slot] = kd[0, 0, j]
    v = _bits(rng.standard_normal((B, H, N, D)))
    dO = _bits(rng.standard_normal((B, H, N, D)))
    t = {n: inputs.to_torch(x, DEV) for n, x in (("q", q), ("k", k), ("v", v), ("dO", dO))}
    f = nss.forward(t["q"], t["k"], t["v"], scale=0.125, causal=True, stabilise=mode, beta=2.0)
    b = nss.backward(t["q"], t["k"], t["v"], f["o"], t["dO"], f["lse"], scale=0.125, causal=True)
    torch.cuda.synchronize()
    ref = oracle.forward(q, k, v, scale=0.125, causal=True, stabilise=mode != 0, beta=2.0)
    rb = oracle.backward(q, k, v, dO, ref, scale=0.125, causal=True)
    parity.check_forward(f, ref, label="negative max mode %d" % mode)
    parity.check_backward(b, rb, label="negative max")
    neg_tie = (ref["ties"] > 1) & (ref["rowmax"] < 0) & (ref["amb_tie"] == 0) & (ref["amb_pbar"] == 0)
    assert neg_tie.sum() > 20
    pone = f["pbar_one"].cpu().numpy()
    if mode:
        assert np.all(pone[neg_tie] == 0)
    else:
        assert np.all(pone[neg_tie] == 1)


@pytest.mark.parametrize("mode", [0, 1])
def test_long_sequence_sampled_rows(mode):
    import numerics_safe_softmax_amd as nss
    w = inputs.custom("long", 1, 2, 32768, 128, True, 91, tie_block=50, v_skew_dims=64, v_mu=-1.5, v_sigma=0.5)
    _say("long sequence N=32768 mode %d" % mode)
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    f = nss.forward(t["q"], t["k"], t["v"], scale=w.scale, causal=True, stabilise=mode, beta=w.beta)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([rng.choice(w.N, 24, replace=False), [0, 1, 127, 128, w.N - 1],
                                   w.N + rng.choice(w.N, 24, replace=False)]))
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=True, stabilise=mode != 0, beta=w.beta,
                         rows=rows, want=parity.FWD_WANT)
    m = np.zeros((1, 2, w.N), dtype=bool)
    m.reshape(-1)[rows] = True
    fr = parity.check_forward(f, ref, rows_mask=m, label="long mode %d" % mode)
    _say("  %s" % fr)


@pytest.mark.parametrize("D,B,H", [(64, 4, 8200), (128, 2, 8200)])
def test_tensors_beyond_2_31_elements(D, B, H):
    import numerics_safe_softmax_amd as nss
    N, mode, G = 1024, 1, 7
    assert B * H * N * D > 2 ** 31
    w = inputs.custom("big", 1, G, N, D, True, 61 + D, tie_block=7, v_skew_dims=D // 4, v_mu=-2.0, v_sigma=0.5,
                      do_mu=-0.5)
    _say("beyond 2^31 elements: B=%d H=%d N=%d D=%d (%d distinct heads)" % (B, H, N, D, G))
    d = inputs.generate(w)
    t = parity.to_dev(d, DEV)
    fs = parity.gpu_forward(t, w, mode)
    bs = parity.gpu_backward(t, w, fs, mode)
    torch.cuda.synchronize()
    ref = oracle.forward(d["q"], d["k"], d["v"], scale=w.scale, causal=True, stabilise=True, beta=w.beta)
    rb = oracle.backward(d["q"], d["k"], d["v"], d["dO"], ref, scale=w.scale, causal=True)
    parity.check_forward(fs, ref, label="seven heads")
    parity.check_backward(bs, rb, label="seven heads")
    idx = torch.arange(B * H, device=DEV) % G
    big = {k: t[k][0].index_select(0, idx).view(B, H, N, D) for k in ("q", "k", "v", "dO")}
    fb = nss.forward(big["q"], big["k"], big["v"], scale=w.scale, causal=True, stabilise=mode, beta=w.beta)
    bb = nss.backward(big["q"], big["k"], big["v"], fb["o"], big["dO"], fb["lse"], scale=w.scale, causal=True,
                      stabilise=mode, beta=w.beta)
    torch.cuda.synchronize()
    _say("  big problem done; comparing every head")
    for name, small, large in (("o", fs["o"], fb["o"]), ("lse", fs["lse"], fb["lse"]),
                               ("ties", fs["ties"], fb["ties"]), ("pbar_one", fs["pbar_one"], fb["pbar_one"]),
                               ("dq", bs["dq"], bb["dq"]), ("dk", bs["dk"], bb["dk"]), ("dv", bs["dv"], bb["dv"]),
                               ("delta", bs["delta"], bb["delta"])):
        want = small[0].index_select(0, idx)
        got = large.reshape(want.shape)
        if want.dtype != torch.int32:
            want, got = want.view(torch.int16 if want.dtype == torch.bfloat16 else torch.int32), \
                got.view(torch.int16 if got.dtype == torch.bfloat16 else torch.int32)
        same = (got == want).reshape(B * H, -1).all(dim=1)
        bad = torch.nonzero(~same).flatten()
        assert bad.numel() == 0, "%s differs in %d heads, first %s" % (name, bad.numel(), bad[:5].tolist())
        del want, got
    del big, fb, bb
    torch.cuda.empty_cache()


# key positions of the repeated maximum, one set per head (the score tile puts
# key offset o of a 32-key block in lane half (o >> 2) & 1)
TIE_KEYS = [(0, 4), (0, 1), (5, 32), (2, 70), (3, 4, 131), (199,)]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_tie_positions_within_and_across_tiles(mode, D, causal):
    import numerics_safe_softmax_amd as nss
    rng = np.random.default_rng(500 + D + 7 * mode + int(causal))
    H, N = len(TIE_KEYS), 200
    q = 0.25 * rng.standard_normal((1, H, N, D))
    q[..., 0] = 1.0
    k = 0.25 * rng.standard_normal((1, H, N, D))
    for h, keys in enumerate(TIE_KEYS):
        for j in keys:
            k[0, h, j, :] = 0.0
            k[0, h, j, 0] = 8.0              # score 8 * scale for every row: far above the rest
    q, k = _bits(q), _bits(k)
    v = _bits(rng.standard_normal((1, H, N, D)))
    dO = _bits(rng.standard_normal((1, H, N, D)))
    t = {n: inputs.to_torch(x, DEV) for n, x in (("q", q), ("k", k), ("v", v), ("dO", dO))}
    scale = D ** -0.5
    f = nss.forward(t["q"], t["k"], t["v"], scale=scale, causal=causal, stabilise=mode, beta=2.0)
    b = nss.backward(t["q"], t["k"], t["v"], f["o"], t["dO"], f["lse"], scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.forward(q, k, v, scale=scale, causal=causal, stabilise=mode != 0, beta=2.0)
    rb = oracle.backward(q, k, v, dO, ref, scale=scale, causal=causal)
    label = "tie keys D%d mode %d causal %d" % (D, mode, causal)
    parity.check_forward(f, ref, label=label)
    parity.check_backward(b, rb, label=label)
    ties = f["ties"].cpu().numpy()[0]
    rows = np.arange(N)
    for h, keys in enumerate(TIE_KEYS):
        # rows that see a copy: the count is the number of copies they see
        want = np.array([sum(1 for j in keys if not causal or j <= i) for i in rows])
        seen = want > 0
        assert np.array_equal(ties[h][seen], want[seen]), (label, keys)
        assert np.array_equal(ref["ties"][0, h][seen], want[seen])
    if mode == 1:
        on = oracle.online_ones(q, k, scale=scale, causal=causal, stabilise=True, beta=2.0,
                               tile=nss.fwd_key_tile(D))
        ok = on["amb"] == 0
        formed = f["formed_ones"].cpu().numpy()
        assert np.array_equal(formed[ok], on["ones"][ok]), label


# The online rule's rescale can grow (itsolotime.com/archives/23922, section
# 极简修复方案, applied to the running (max, count) pair): a maximum repeated
# in an early KV tile moves the shift to beta * rm (rm > 0) or to 0 (rm < 0);
# a later, larger single maximum that stays below beta * rm (or below 0)
# brings the shift back down to itself, so the rescale factor
# alpha = exp(shift_old - shift_new) exceeds 1.  Per head: the repeated keys,
# their raw score, the overtaking key and its raw score (q_i = e_0 plus a
# small second component, so the marked keys score exactly their value).
R10_HEADS = [
    ((10, 40), 4.0, 150, 6.0),     # positive: shift 8 -> 6 (alpha = e^(2 scale))
    ((10, 70), 4.0, 150, 7.5),     # the repeat completes in tile 1 (shift up), then down in tile 2
    ((10, 40), -1.0, 150, -0.5),   # negative: shift 0 -> -0.5
    ((3, 60), -2.0, 100, -1.25),   # negative, overtaken in the next 64-key tile
]


def _online_shifts(raw, beta, tile):
    """The rule's shift after each tile of one row (exact small numbers)."""
    out, m, c = [], -np.inf, 0
    for t0 in range(0, len(raw), tile):
        seg = raw[t0:t0 + tile]
        mx = max(seg)
        cnt = sum(1 for x in seg if x == mx)
        if mx > m:
            m, c = mx, cnt
        elif mx == m:
            c += cnt
        out.append(beta * m if c > 1 and m > 0 else (0.0 if c > 1 and m < 0 else m))
    return out


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_online_shift_moves_down(mode, D, causal):
    import numerics_safe_softmax_amd as nss
    rng = np.random.default_rng(700 + D + 3 * mode + int(causal))
    H, N, beta = len(R10_HEADS), 200, 2.0
    q = np.zeros((1, H, N, D))
    q[..., 0] = 1.0
    q[..., 1] = 0.25 * rng.standard_normal((1, H, N))
    k = np.zeros((1, H, N, D))
    k[..., 1] = 0.25 * rng.standard_normal((1, H, N))
    for h, (reps, a, b, bval) in enumerate(R10_HEADS):
        # the other keys score well below the marked ones
        low = min(a, bval) - 3.0
        k[0, h, :, 0] = low - 0.25 * np.abs(rng.standard_normal(N))
        for j in reps:
            k[0, h, j, :2] = (a, 0.0)
        k[0, h, b, :2] = (bval, 0.0)
    q, k = _bits(q), _bits(k)
    v = rng.standard_normal((1, H, N, D))
    v[..., :16] = -2.0 + 0.5 * rng.standard_normal((1, H, N, 16))
    v, dO = _bits(v), _bits(rng.standard_normal((1, H, N, D)))
    scale = D ** -0.5
    # the construction: on the rows that see every marked key the running shift
    # rises at the repeat and falls at the overtaking key
    T = nss.fwd_key_tile(D)
    for h, (reps, a, b, bval) in enumerate(R10_HEADS):
        raw = inputs.bits_to_float(k[0, h, :, 0]).astype(np.float64)
        sh = _online_shifts(list(raw), beta, T)
        assert sh[b // T] < sh[b // T - 1], (h, sh)
    t = {n: inputs.to_torch(x, DEV) for n, x in (("q", q), ("k", k), ("v", v), ("dO", dO))}
    label = "shift moves down D%d mode %d causal %d" % (D, mode, causal)
    _say(label)
    f = nss.forward(t["q"], t["k"], t["v"], scale=scale, causal=causal, stabilise=mode, beta=beta)
    b = nss.backward(t["q"], t["k"], t["v"], f["o"], t["dO"], f["lse"], scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.forward(q, k, v, scale=scale, causal=causal, stabilise=mode != 0, beta=beta)
    rb = oracle.backward(q, k, v, dO, ref, scale=scale, causal=causal)
    parity.check_forward(f, ref, label=label)
    parity.check_backward(b, rb, label=label)
    ties = f["ties"].cpu().numpy()[0]
    for h, (reps, a, bkey, bval) in enumerate(R10_HEADS):
        seen_b = np.arange(N) >= bkey if causal else np.ones(N, dtype=bool)
        assert np.all(ties[h][seen_b] == 1), label          # the overtaking key is the single maximum
    if mode in (0, 1):
        on = oracle.online_ones(q, k, scale=scale, causal=causal, stabilise=mode == 1, beta=beta,
                               tile=nss.fwd_key_tile(D))
        ok = on["amb"] == 0
        assert np.array_equal(f["formed_ones"].cpu().numpy()[ok], on["ones"][ok]), label
    else:
        exn = (ref["amb_tie"] == 0) & (ref["amb_near"] == 0)
        assert np.array_equal(f["formed_ones"].cpu().numpy()[exn], ref["near_ones"][exn]), label
