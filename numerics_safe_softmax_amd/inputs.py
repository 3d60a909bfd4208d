"""Seeded synthetic workloads: bf16 Q, K, V, dO with injected duplicate-max rows.

This module is the ONE piece both sides share: the HIP path (tests, bench) and
the FP64 oracle (tests) receive the same bf16 bit patterns from it.  It holds
none of the method's arithmetic -- no softmax, no shift rule, no tie counting.
It draws normal / ternary values with numpy's PCG64, converts them to bf16 by
round-to-nearest-even, and builds the duplicate-max rows the workloads ask for
by copying key vectors (the argmax of one float64 dot-product row picks which
key to copy).

The workloads stand in for the pages' setting: GPT-2 small / medium attention
(12 layers, 12 heads, d_model 768, context 1024; itsolotime.com/archives/23922,
section "核心发现" and section "实验结果"), rows whose score maximum repeats
(same page, section "机制解释二", the trigger) and value dimensions dominated by
negative numbers (same section, the bias source).  No dataset item is used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    causal: bool
    seed: int
    tie_block: int = 0          # one duplicate-max row per this many rows (0 = none)
    v_skew_dims: int = 0        # the first dims of V drawn from N(v_mu, v_sigma)
    v_mu: float = 0.0
    v_sigma: float = 1.0
    do_mu: float = 0.0          # dO ~ N(do_mu, 1)
    sink: bool = False          # ternary Q/K with an attention-sink key (non-causal)
    beta: float = 2.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def visible_pairs(self) -> int:
        per_head = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return self.B * self.H * per_head

    def fwd_flops(self) -> float:
        """Algorithmic forward flops: 4 D per visible (query, key) pair."""
        return 4.0 * self.D * self.visible_pairs()

    def bwd_flops(self) -> float:
        """Algorithmic backward flops: 10 D per visible pair (S recompute, dP, dV, dK, dQ)."""
        return 10.0 * self.D * self.visible_pairs()


# The five workloads: a tiny single head, GPT-2 small and medium attention
# layers, a long-context layer and a tie-heavy attention-sink stress case.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 1, 128, 64, True, 1, tie_block=4, v_skew_dims=16, v_mu=-2.0,
                     v_sigma=0.5, do_mu=0.0),
    "gpt2_small": Workload("gpt2_small", 8, 12, 1024, 64, True, 2, tie_block=10, v_skew_dims=16,
                           v_mu=-2.0, v_sigma=0.5, do_mu=-0.5),
    "gpt2_medium": Workload("gpt2_medium", 8, 16, 1024, 64, True, 3, tie_block=10, v_skew_dims=16,
                            v_mu=-2.0, v_sigma=0.5, do_mu=-0.5),
    "long_context": Workload("long_context", 1, 16, 8192, 128, True, 4, tie_block=20,
                             v_skew_dims=64, v_mu=-1.5, v_sigma=0.5, do_mu=0.0),
    "sink": Workload("sink", 4, 12, 2048, 64, False, 5, v_skew_dims=32, v_mu=-2.0, v_sigma=0.5,
                     do_mu=-0.5, sink=True),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest even (normal range only)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)
    sign = (r >> np.uint64(18)) & np.uint64(1)
    e11 = ((r >> np.uint64(7)) & np.uint64(0x7FF)).astype(np.int64)
    frac = r & np.uint64(0x7F)
    zero = x == 0.0
    e8 = e11 - 1023 + 127
    if np.any((~zero) & ((e8 < 1) | (e8 > 254))):
        raise ValueError("value outside the bf16 normal range")
    bits = (sign << np.uint64(15)) | (np.where(zero, 0, e8).astype(np.uint64) << np.uint64(7)) | \
        np.where(zero, np.uint64(0), frac)
    return bits.astype(np.uint16)


def bits_to_float(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _inject_ties(q: np.ndarray, k: np.ndarray, block: int, rng: np.random.Generator) -> np.ndarray:
    """Copy key vectors so that one query row per ``block`` has its max twice.

    For head (b, h), the targets are one row per block of ``block`` rows, at
    offset 2..block-1 inside the block.  Targets are visited in order; for
    target i, with i_prev the previous target, the key j* scoring highest
    against q_i (j* <= i) is copied into a position j' drawn from
    (i_prev, i) minus {j*}.  j' < i keeps the copy visible to row i under the
    causal mask, and j' > i_prev leaves every earlier target's row untouched,
    so each target ends with its maximum at least twice.
    """
    B, H, N, D = q.shape
    qf = bits_to_float(q).astype(np.float64)
    kf = bits_to_float(k).astype(np.float64)
    out = k.copy()
    nblocks = N // block
    for b in range(B):
        for h in range(H):
            if nblocks == 0:
                continue
            offs = rng.integers(2, block, size=nblocks)
            targets = np.arange(nblocks) * block + offs
            picks = rng.random(size=nblocks)
            scores = qf[b, h, targets] @ kf[b, h].T          # [T, N] against the original keys
            cur = np.arange(N)                                # which original key each slot holds
            prev = -1
            for t, i in enumerate(targets):
                row = scores[t, cur[: i + 1]]
                jstar = int(np.argmax(row))
                cand = [j for j in range(prev + 1, i) if j != jstar]
                jp = cand[min(int(picks[t] * len(cand)), len(cand) - 1)]
                cur[jp] = cur[jstar]
                prev = int(i)
            out[b, h] = k[b, h][cur]
    return out


def generate(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """bf16 bit patterns (uint16, [B, H, N, D]) of q, k, v, dO for a workload."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, H, N, D = w.B, w.H, w.N, w.D
    shape = (B, H, N, D)
    if w.sink:
        half = D // 2
        tern = np.array([-0.5, 0.0, 0.5])
        q = np.empty(shape)
        q[..., :half] = 0.5                                   # channel shared by every query
        q[..., half:] = tern[rng.integers(0, 3, size=(B, H, N, D - half))]
        k = np.empty(shape)
        k[..., :half] = 0.0
        k[..., half:] = tern[rng.integers(0, 3, size=(B, H, N, D - half))]
        k[:, :, 0, :half] = 0.5                               # key 0: the sink
        k[:, :, 0, half:] = 0.0
    else:
        q = rng.standard_normal(shape)
        k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    if w.v_skew_dims:
        v[..., : w.v_skew_dims] = w.v_mu + w.v_sigma * rng.standard_normal(
            (B, H, N, w.v_skew_dims))
    dO = w.do_mu + rng.standard_normal(shape)
    qb, kb, vb, gb = (to_bf16_bits(a) for a in (q, k, v, dO))
    if w.sink:
        for b in range(B):                                    # three copies of the sink key
            pos = rng.choice(np.arange(1, N), size=min(3, N - 1), replace=False)  # fewer when N < 4
            for j in pos:
                kb[b, :, j, :] = kb[b, :, 0, :]
    elif w.tie_block and w.causal:
        kb = _inject_ties(qb, kb, w.tie_block, rng)
    return {"q": qb, "k": kb, "v": vb, "dO": gb}


def custom(name: str, B: int, H: int, N: int, D: int, causal: bool, seed: int, **kw) -> Workload:
    """A workload of any shape with the same recipe (for parity sweeps)."""
    return Workload(name, B, H, N, D, causal, seed, **kw)


def to_torch(bits: np.ndarray, device=None):
    """bf16 bit patterns -> a torch.bfloat16 tensor (optionally moved to a device)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t
