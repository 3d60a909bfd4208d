"""HIP-graph capture of the whole path (attn_fwd + attn_bwd) on the GPU.

The library allocates nothing, never synchronises and records no memset, so a
forward + backward can be captured once and replayed.  Each replay is checked
bit for bit against the eager result, with eager work and synchronisations
between the replays and the graph's outputs overwritten before each one (a
replay that skipped a kernel would leave the overwritten values behind).
"""
import pytest

from numerics_safe_softmax_amd import inputs
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _buffers(q):
    B, H, N, D = q.shape
    rows = lambda dt: torch.empty((B, H, N), dtype=dt, device=q.device)
    return {"o": torch.empty_like(q), "lse": rows(torch.float32), "ties": rows(torch.int32),
            "pone": rows(torch.int32), "formed": rows(torch.int32), "dq": torch.empty_like(q),
            "dk": torch.empty_like(q), "dv": torch.empty_like(q), "delta": rows(torch.float32)}


def _step(nss, t, b, w, mode, stream):
    kw = dict(scale=w.scale, causal=w.causal, stream=stream)
    nss.attn_fwd(t["q"], t["k"], t["v"], b["o"], b["lse"], b["ties"], b["pone"], b["formed"], stabilise=mode,
                 beta=w.beta, **kw)
    nss.attn_bwd(t["q"], t["k"], t["v"], b["o"], t["dO"], b["lse"], b["dq"], b["dk"], b["dv"], b["delta"],
                 stabilise=mode, beta=w.beta, **kw)


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


# (B, H, N, D, modes): a small grid in every mode, and a grid whose dK/dV key
# tiles are paired and placed (72 key tiles per XCD; the placement is a
# by-value kernel argument, copied into the graph at capture)
GRAPH_CASES = [(1, 8, 640, 64, m) for m in (0, 1, 2)] + [(1, 96, 650, 64, 1)]
# d = 128: 32-key forward tiles at three workgroups per CU, 32-query dK/dV tiles
GRAPH_CASES += [(1, 8, 700, 128, m) for m in (1, 2)]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=lambda c: "B%dH%dN%dD%d_m%d" % c)
def test_graph_replays_match_eager(case):
    import numerics_safe_softmax_amd as nss
    B, H, N, D, mode = case
    w = inputs.custom("graph", B, H, N, D, True, 31, tie_block=8, v_skew_dims=16, v_mu=-2.0, v_sigma=0.5,
                      do_mu=-0.5)
    print("graph %s" % (case,), flush=True)
    t = parity.to_dev(inputs.generate(w), DEV)
    eager = _buffers(t["q"])
    graph = _buffers(t["q"])
    main = torch.cuda.current_stream()
    _step(nss, t, eager, w, mode, main)
    torch.cuda.synchronize()
    ref = {k: x.clone() for k, x in eager.items()}

    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        _step(nss, t, graph, w, mode, side)  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        _step(nss, t, graph, w, mode, side)
    torch.cuda.synchronize()

    for rep in range(3):
        for x in graph.values():
            x.fill_(-7 if x.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert _same(graph[k], ref[k]), "replay %d: %s differs from the eager result" % (rep, k)
        # eager work between replays, into the eager buffers
        _step(nss, t, eager, w, mode, main)
        torch.cuda.synchronize()
        for k in ref:
            assert _same(eager[k], ref[k]), "eager rerun %d: %s changed" % (rep, k)
