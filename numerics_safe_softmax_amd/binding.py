"""ctypes binding of libattn.so (include/attn.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
data pointers, shapes and the current HIP stream to the C entry point of the
same name, and raises AttnError on a non-zero status.  All arithmetic runs in
the library's gfx950 kernels; there is no fallback path.  If libattn.so has
not been built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "attn.h")

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

_SIGS = {
    "attn_fwd": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _F, _P],
    "attn_fwd_o32": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _I, _F, _P],
    "attn_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _F, _I, _I, _F, _P],
    "attn_bwd_o32": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _I, _F, _I, _I, _F, _P],
    "attn_bwd_workspace_bytes": [_I, _I, _I, _I],
    "attn_bwd_dq": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P],
    "attn_bwd_dkdv": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P],
    "attn_tiecount": [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P],
    "attn_status_string": [_I],
    "attn_abi_version": [],
    "attn_fwd_key_tile": [_I],
}


class AttnError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__("attn status %d: %s" % (status, text))
        self.status = status


_lib = None


def lib():
    """Load libattn.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libattn.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = {"attn_status_string": ctypes.c_char_p,
                         "attn_bwd_workspace_bytes": ctypes.c_size_t}.get(name, ctypes.c_int)
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions declared in include/attn.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().attn_abi_version())


def fwd_key_tile(D: int) -> int:
    """Keys per KV tile of the forward for head size D (the online modes'
    tile-by-tile shift depends on it)."""
    w = int(lib().attn_fwd_key_tile(int(D)))
    _check(min(w, 0))
    return w


def _check(rc: int) -> None:
    if rc != 0:
        raise AttnError(rc, status_string(rc))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the C ABI must be contiguous")
    if not t.is_cuda:
        # the library dereferences device pointers only; a host pointer would fault the GPU
        raise ValueError("tensors passed to the C ABI must live on the GPU (got %s)" % t.device)
    return t.data_ptr() or None


def _expect(t, dtype, shape, name):
    """dtype / shape check of one argument (None passes: optional outputs)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check_args(q, mats=(), rows=(), ints=()):
    """bf16 [B, H, N, D] matrices, fp32 and int32 [B, H, N] row vectors, one device."""
    import torch
    B, H, N, D = _shape(q)
    _expect(q, torch.bfloat16, (B, H, N, D), "q")
    for name, t in mats:
        _expect(t, torch.bfloat16, (B, H, N, D), name)
    for name, t in rows:
        _expect(t, torch.float32, (B, H, N), name)
    for name, t in ints:
        _expect(t, torch.int32, (B, H, N), name)
    for name, t in list(mats) + list(rows) + list(ints):
        if t is not None and t.device != q.device:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, q.device))
    return B, H, N, D


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


PLAIN, STAB_ONLINE, STAB_EXACT = 0, 1, 2


def _mode(stabilise) -> int:
    """stabilise: False/0 plain, True/1 online duplicate-max shift, 2 exact final shift."""
    return int(stabilise)


def _shape(q):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, D]")
    return tuple(int(x) for x in q.shape)


def attn_fwd(q, k, v, o, lse, ties=None, pbar_one=None, formed_ones=None, *, scale: float,
             causal: bool, stabilise: bool, beta: float = 2.0, stream=None) -> None:
    B, H, N, D = _check_args(q, mats=(("k", k), ("v", v), ("o", o)), rows=(("lse", lse),),
                             ints=(("ties", ties), ("pbar_one", pbar_one), ("formed_ones", formed_ones)))
    _check(lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ties), _ptr(pbar_one),
                          _ptr(formed_ones), B, H, N, D, float(scale), int(bool(causal)),
                          _mode(stabilise), float(beta), _stream(stream)))


def attn_fwd_o32(q, k, v, o, o32, lse, ties=None, pbar_one=None, formed_ones=None, *, scale: float,
                 causal: bool, stabilise: bool, beta: float = 2.0, stream=None) -> None:
    import torch
    B, H, N, D = _check_args(q, mats=(("k", k), ("v", v), ("o", o)), rows=(("lse", lse),),
                             ints=(("ties", ties), ("pbar_one", pbar_one), ("formed_ones", formed_ones)))
    _expect(o32, torch.float32, (B, H, N, D), "o32")
    _check(lib().attn_fwd_o32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o32), _ptr(lse), _ptr(ties),
                              _ptr(pbar_one), _ptr(formed_ones), B, H, N, D, float(scale), int(bool(causal)),
                              _mode(stabilise), float(beta), _stream(stream)))


def attn_bwd_workspace_bytes(B: int, H: int, N: int, D: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(int(B), int(H), int(N), int(D)))


def _ws(workspace):
    """(pointer, bytes) of a workspace tensor (any dtype, on the GPU), or (None, 0)."""
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def attn_bwd_o32(q, k, v, o32, dO, lse, dq, dk, dv, delta, workspace=None, *, scale: float, causal: bool,
                 stabilise: bool, beta: float = 2.0, stream=None) -> None:
    import torch
    B, H, N, D = _check_args(q, mats=(("k", k), ("v", v), ("dO", dO), ("dq", dq), ("dk", dk), ("dv", dv)),
                             rows=(("lse", lse), ("delta", delta)))
    _expect(o32, torch.float32, (B, H, N, D), "o32")
    wp, wb = _ws(workspace)
    _check(lib().attn_bwd_o32(_ptr(q), _ptr(k), _ptr(v), _ptr(o32), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), _ptr(delta), wp, wb, B, H, N, D, float(scale), int(bool(causal)),
                              _mode(stabilise), float(beta), _stream(stream)))


def attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, delta, workspace=None, *, scale: float, causal: bool,
             stabilise: bool, beta: float = 2.0, stream=None) -> None:
    B, H, N, D = _check_args(q, mats=(("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq), ("dk", dk),
                                      ("dv", dv)), rows=(("lse", lse), ("delta", delta)))
    wp, wb = _ws(workspace)
    _check(lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(delta), wp, wb, B, H, N, D, float(scale), int(bool(causal)),
                          _mode(stabilise), float(beta), _stream(stream)))


def attn_bwd_dq(q, k, v, o, dO, lse, dq, delta, *, scale: float, causal: bool, stream=None) -> None:
    B, H, N, D = _check_args(q, mats=(("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq)),
                             rows=(("lse", lse), ("delta", delta)))
    _check(lib().attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq),
                             _ptr(delta), B, H, N, D, float(scale), int(bool(causal)), _stream(stream)))


def attn_bwd_dkdv(q, k, v, dO, lse, delta, dk, dv, *, scale: float, causal: bool, stream=None) -> None:
    B, H, N, D = _check_args(q, mats=(("k", k), ("v", v), ("dO", dO), ("dk", dk), ("dv", dv)),
                             rows=(("lse", lse), ("delta", delta)))
    _check(lib().attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(delta), _ptr(dk),
                               _ptr(dv), B, H, N, D, float(scale), int(bool(causal)), _stream(stream)))


def attn_tiecount(q, k, ties, rowmax=None, *, scale: float, causal: bool, stream=None) -> None:
    B, H, N, D = _check_args(q, mats=(("k", k),), rows=(("rowmax", rowmax),), ints=(("ties", ties),))
    _check(lib().attn_tiecount(_ptr(q), _ptr(k), _ptr(ties), _ptr(rowmax), B, H, N, D, float(scale),
                               int(bool(causal)), _stream(stream)))


# ------------------------------------------------------------- conveniences
# Allocation of outputs with torch, then one call of the entry point above.

def forward(q, k, v, *, scale: float, causal: bool, stabilise: bool, beta: float = 2.0,
            diagnostics: bool = True, o32: bool = False, stream=None) -> dict:
    """attn_fwd (or attn_fwd_o32 with o32=True, adding the fp32 O as "o32")."""
    import torch
    B, H, N, D = _shape(q)
    dev = q.device
    out = {"o": torch.empty_like(q), "lse": torch.empty((B, H, N), dtype=torch.float32, device=dev)}
    if diagnostics:
        for f in ("ties", "pbar_one", "formed_ones"):
            out[f] = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    if o32:
        out["o32"] = torch.empty((B, H, N, D), dtype=torch.float32, device=dev)
        attn_fwd_o32(q, k, v, out["o"], out["o32"], out["lse"], out.get("ties"), out.get("pbar_one"),
                     out.get("formed_ones"), scale=scale, causal=causal, stabilise=stabilise, beta=beta,
                     stream=stream)
    else:
        attn_fwd(q, k, v, out["o"], out["lse"], out.get("ties"), out.get("pbar_one"), out.get("formed_ones"),
                 scale=scale, causal=causal, stabilise=stabilise, beta=beta, stream=stream)
    return out


def workspace_for(q):
    """A workspace tensor of attn_bwd_workspace_bytes for q's shape (None when 0)."""
    import torch
    nb = attn_bwd_workspace_bytes(*_shape(q))
    return torch.empty(nb // 4, dtype=torch.float32, device=q.device) if nb else None


def backward(q, k, v, o, dO, lse, *, scale: float, causal: bool, stabilise: bool = False,
             beta: float = 2.0, o32=None, workspace=None, stream=None) -> dict:
    """attn_bwd (or attn_bwd_o32 when the fp32 O is given: delta from it); the
    workspace is allocated here unless one is passed."""
    import torch
    B, H, N, D = _shape(q)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(q), "dv": torch.empty_like(q),
           "delta": torch.empty((B, H, N), dtype=torch.float32, device=q.device)}
    ws = workspace if workspace is not None else workspace_for(q)
    if o32 is not None:
        attn_bwd_o32(q, k, v, o32, dO, lse, out["dq"], out["dk"], out["dv"], out["delta"], ws, scale=scale,
                     causal=causal, stabilise=stabilise, beta=beta, stream=stream)
    else:
        attn_bwd(q, k, v, o, dO, lse, out["dq"], out["dk"], out["dv"], out["delta"], ws, scale=scale,
                 causal=causal, stabilise=stabilise, beta=beta, stream=stream)
    return out


def tiecount(q, k, *, scale: float, causal: bool, stream=None) -> dict:
    import torch
    B, H, N, D = _shape(q)
    out = {"ties": torch.empty((B, H, N), dtype=torch.int32, device=q.device),
           "rowmax": torch.empty((B, H, N), dtype=torch.float32, device=q.device)}
    attn_tiecount(q, k, out["ties"], out["rowmax"], scale=scale, causal=causal, stream=stream)
    return out
