"""torch.autograd entry to the fused attention, and a GPT-2-shaped attention
layer built on it.

``attention(q, k, v)`` runs ``attn_fwd`` in the forward and ``attn_bwd`` in
the backward of a ``torch.autograd.Function``; both are the library's gfx950
kernels (this module only allocates outputs and passes pointers).  The saved
state is Q, K, V, O and the per-row log-sum-exp, as the backward recomputes
P = exp(S - LSE) from them (FlashAttention's recomputation).

``GPT2Attention`` is one attention sublayer of GPT-2 small (d_model 768, 12
heads of 64, causal), the setting of Qiu & Yao's experiments as summarised on
itsolotime.com/archives/23922 (section 核心发现): a fused QKV projection,
the attention above, an output projection.  Its two projections are plain
bf16 matrix products left to torch (hipBLASLt); they are outside the hot path.
Weights are random (N(0, 0.02), zero biases, as GPT-2 initialises them); no
trained weights or data are used.
"""
from __future__ import annotations

import math

import torch

from . import binding


class _FusedAttention(torch.autograd.Function):

    @staticmethod
    def forward(ctx, q, k, v, scale, causal, stabilise, beta):
        out = binding.forward(q, k, v, scale=scale, causal=causal, stabilise=stabilise, beta=beta,
                              diagnostics=False)
        ctx.save_for_backward(q, k, v, out["o"], out["lse"])
        ctx.cfg = (scale, causal, stabilise, beta)
        return out["o"]

    @staticmethod
    def backward(ctx, dO):
        q, k, v, o, lse = ctx.saved_tensors
        scale, causal, stabilise, beta = ctx.cfg
        g = binding.backward(q, k, v, o, dO.contiguous(), lse, scale=scale, causal=causal,
                             stabilise=stabilise, beta=beta)
        return g["dq"], g["dk"], g["dv"], None, None, None, None


def attention(q, k, v, *, scale=None, causal: bool = True, stabilise=1, beta: float = 2.0):
    """Softmax attention of bf16 [B, H, N, D] tensors on the GPU, differentiable.

    stabilise: 0 plain, 1 online duplicate-max shift, 2 exact final shift.
    scale defaults to 1/sqrt(D).  Inputs must be contiguous; there is no CPU
    path (the binding raises for host tensors).
    """
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _FusedAttention.apply(q, k, v, float(scale), bool(causal), int(stabilise), float(beta))


class GPT2Attention(torch.nn.Module):
    """GPT-2 attention sublayer: x [B, T, C] -> x [B, T, C], C = n_head * 64."""

    def __init__(self, d_model: int = 768, n_head: int = 12, *, stabilise=1, beta: float = 2.0,
                 device=None, seed: int = 0):
        super().__init__()
        if d_model % n_head:
            raise ValueError("d_model must be a multiple of n_head")
        self.d_model, self.n_head, self.head_dim = d_model, n_head, d_model // n_head
        self.stabilise, self.beta = stabilise, beta
        gen = torch.Generator(device="cpu").manual_seed(seed)

        def param(*shape, std):
            w = torch.randn(*shape, generator=gen) * std if std else torch.zeros(*shape)
            return torch.nn.Parameter(w.to(device=device, dtype=torch.bfloat16))

        self.w_qkv = param(3 * d_model, d_model, std=0.02)
        self.b_qkv = param(3 * d_model, std=0.0)
        self.w_out = param(d_model, d_model, std=0.02)
        self.b_out = param(d_model, std=0.0)
        self.last_qkv = None  # the attention inputs of the latest forward, for diagnostics
        self.last_o = None    # its output (with .grad after backward)

    def forward(self, x):
        B, T, C = x.shape
        qkv = torch.nn.functional.linear(x.reshape(B * T, C), self.w_qkv, self.b_qkv)
        qkv = qkv.reshape(B, T, 3, self.n_head, self.head_dim).permute(2, 0, 3, 1, 4).contiguous()
        q, k, v = qkv[0], qkv[1], qkv[2]
        self.last_qkv = (q.detach(), k.detach(), v.detach())
        o = attention(q, k, v, causal=True, stabilise=self.stabilise, beta=self.beta)
        if o.requires_grad:
            o.retain_grad()  # dL/dO of the attention, for diagnostics
        self.last_o = o
        y = o.transpose(1, 2).reshape(B * T, C)
        return torch.nn.functional.linear(y, self.w_out, self.b_out).reshape(B, T, C)
