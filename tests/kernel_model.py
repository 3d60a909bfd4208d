"""A numpy model of the GPU kernels' arithmetic, independent of the oracle.

TEST HELPER.  It exists to pin the oracle's tolerance tensors from the other
side: an implementation that does what the kernels do -- bf16 operands, fp32
products and sums, P_bar formed in fp32 and rounded to bf16 (nearest even)
for P_bar V, O normalised by the sum of those bf16 values, LSE from the sum
of the fp32 values, the duplicate-max rule applied to the running (max,
count) pair tile by tile, bf16 outputs -- must land inside the tolerances,
and plausible mistakes must land outside.  It imports nothing from
``oracle/`` and nothing from the HIP package; the only shared piece is the
seeded input generator.

What it follows (web pages on Qiu & Yao, "Why Low-Precision Transformer
Training Fails: An Analysis on Flash Attention"):
* itsolotime.com/archives/23922, section 机制解释二: P_bar = exp(S - m),
  P = P_bar / rowsum(P_bar), O = P V, with P_bar in BF16 as the operand of
  P_bar V.
* same page, section 极简修复方案: the row maximum's repeat count, and the shift
  beta * rm (repeated, rm > 0), 0 (repeated, rm < 0) or rm (otherwise).
* 91haoming.cn/news/show-608006, section 三: delta_i = sum_c dO_ic O_ic; then
  dP = dO V^T, dS = P o (dP - delta) and the three gradient products.

The order of fp32 additions differs from the kernels' (numpy's blocked sums
against MFMA chains); any order is a legitimate fp32 computation, which is the
point: the tolerances must hold for all of them.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
LOG2E = F32(1.4426950408889634)
LN2 = F32(0.6931471805599453)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _fma32(a: np.ndarray, b: F32, c: np.ndarray) -> np.ndarray:
    """fl32(a * b + c) with one rounding: the float64 product of two float32
    values is exact, and one float64 addition before the float32 rounding
    leaves the result within an ulp of the fused value."""
    return (a.astype(np.float64) * np.float64(b) + c.astype(np.float64)).astype(np.float32)


def _shift(m: np.ndarray, c: np.ndarray, base: np.ndarray, stabilise: bool, beta: F32) -> np.ndarray:
    """The duplicate-max rule on (max, count), in the log2-scaled units of base = m * scale * log2 e."""
    out = base.copy()
    if stabilise:
        rep = c > 1
        out = np.where(rep & (m > 0), beta * base, out)
        out = np.where(rep & (m < 0), F32(0), out)
    return out.astype(np.float32)


def _visible(N: int, k0: int, k1: int, causal: bool) -> np.ndarray:
    rows = np.arange(N)[:, None]
    keys = np.arange(k0, k1)[None, :]
    return (keys <= rows) if causal else np.ones((N, k1 - k0), dtype=bool)


def forward_head(q, k, v, scale: float, causal: bool, mode: int, beta: float = 2.0, tile: int = 64,
                 row_sum: str = "bf16") -> dict:
    """One head: q, k, v bf16 bits [N][D].  mode 0 plain, 1 online shift,
    2 shift from each row's final (max, count).  row_sum: what O is divided
    by -- "bf16", the sum of the rounded P_bar that P_bar V consumes (the
    kernels), or "fp32", the sum of the unrounded values (a reading the
    tests use as a control).  Returns O (bf16 values as float32), LSE
    (float32) and the duplicate counts."""
    Q, K, V = bits_to_f32(q), bits_to_f32(k), bits_to_f32(v)
    N, D = Q.shape
    t = F32(scale) * LOG2E
    beta = F32(beta)
    # the whole row's (max, count), for mode 2
    full = Q @ K.T
    full = np.where(_visible(N, 0, N, causal), full, -np.inf).astype(np.float32)
    rm = full.max(axis=1)
    rs = (full == rm[:, None]).sum(axis=1)
    final_m2 = _shift(rm, rs, rm * t, mode != 0, beta)

    m_run = np.full(N, -np.inf, dtype=np.float32)
    c_run = np.zeros(N, dtype=np.int64)
    m2_run = np.full(N, -np.inf, dtype=np.float32)
    lsum = np.zeros(N, dtype=np.float32)
    lsum_bf = np.zeros(N, dtype=np.float32)
    oacc = np.zeros((N, D), dtype=np.float32)
    for k0 in range(0, N, tile):
        k1 = min(N, k0 + tile)
        s = (Q @ K[k0:k1].T).astype(np.float32)
        s = np.where(_visible(N, k0, k1, causal), s, -np.inf).astype(np.float32)
        mx = s.max(axis=1)
        cnt = (s == mx[:, None]).sum(axis=1)
        cnt = np.where(mx == -np.inf, 0, cnt)
        up = mx > m_run
        c_run = np.where(up, cnt, np.where(mx == m_run, c_run + cnt, c_run))
        m_run = np.where(up, mx, m_run)
        m2 = final_m2 if mode == 2 else _shift(m_run, c_run, (m_run * t).astype(np.float32), mode == 1, beta)
        seen = m_run > -np.inf
        alpha = np.where(m2_run == -np.inf, F32(0), np.exp2((m2_run - m2).astype(np.float32)))
        alpha = np.where(seen, alpha, F32(0)).astype(np.float32)
        m2_run = np.where(seen, m2, m2_run).astype(np.float32)
        lsum = (lsum * alpha).astype(np.float32)
        lsum_bf = (lsum_bf * alpha).astype(np.float32)
        oacc = (oacc * alpha[:, None]).astype(np.float32)
        x = _fma32(s, t, -np.where(seen, m2, F32(0))[:, None])
        p = np.exp2(x).astype(np.float32)
        p = np.where(np.isfinite(s), p, F32(0)).astype(np.float32)
        pb = round_bf16(p)
        lsum = (lsum + p.sum(axis=1, dtype=np.float32)).astype(np.float32)
        lsum_bf = (lsum_bf + pb.sum(axis=1, dtype=np.float32)).astype(np.float32)
        oacc = (oacc + pb @ V[k0:k1]).astype(np.float32)
    inv = (F32(1) / (lsum_bf if row_sum == "bf16" else lsum)).astype(np.float32)
    O = round_bf16((oacc * inv[:, None]).astype(np.float32))
    lse = ((m2_run + np.log2(lsum).astype(np.float32)) * LN2).astype(np.float32)
    return {"O": O, "lse": lse, "ties": c_run, "rowmax": rm * F32(scale)}


def backward_head(q, k, v, dO, O, lse, scale: float, causal: bool) -> dict:
    """One head's backward from the forward's bf16 O and fp32 LSE: delta,
    P = exp(S - LSE), dP = dO V^T, dS = P (dP - delta), dV = P^T dO,
    dK = scale dS^T Q, dQ = scale dS K, with P and dS rounded to bf16 as
    product operands and bf16 results."""
    Q, K, V, G = bits_to_f32(q), bits_to_f32(k), bits_to_f32(v), bits_to_f32(dO)
    N, D = Q.shape
    t = F32(scale) * LOG2E
    delta = (G * O).sum(axis=1, dtype=np.float32)
    lse2 = (lse * LOG2E).astype(np.float32)
    s = (Q @ K.T).astype(np.float32)
    vis = _visible(N, 0, N, causal)
    P = np.exp2(_fma32(s, t, -lse2[:, None])).astype(np.float32)
    P = np.where(vis, P, F32(0)).astype(np.float32)
    dP = (G @ V.T - delta[:, None]).astype(np.float32)
    dS = (P * dP).astype(np.float32)
    Pb, dSb = round_bf16(P), round_bf16(dS)
    dV = round_bf16((Pb.T @ G).astype(np.float32))
    dK = round_bf16(((dSb.T @ Q) * F32(scale)).astype(np.float32))
    dQ = round_bf16(((dSb @ K) * F32(scale)).astype(np.float32))
    return {"delta": delta, "dQ": dQ, "dK": dK, "dV": dV}
