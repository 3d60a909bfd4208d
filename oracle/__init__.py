"""FP64 CPU oracle for BF16 softmax attention with the duplicate-max shift.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``numerics_safe_softmax_amd``) and imports nothing
from it; both sides take their inputs from the seeded generator module.

The arithmetic lives in ``oracle.c`` (plain C, FP64, OpenMP over rows); this
module only marshals numpy arrays.  Pages followed (Qiu & Yao, "Why
Low-Precision Transformer Training Fails: An Analysis on Flash Attention"):

* itsolotime.com/archives/23922, section "机制解释二" (origin of the bias):
  P_bar = exp(S - m), P = P_bar / rowsum(P_bar), O = P V.
* same page, section "极简修复方案" (minimal fix): count how often the row max
  occurs; if it repeats, shift by beta * max (max > 0) or by 0 (max < 0),
  else by the max.
* 91haoming.cn/news/show-608006, section 三: delta is a row-sum of an
  element-wise product (delta_i = sum_c dO_ic O_ic); section 四: the worked
  bf16 addition of -2.40625 and -2.296875.

Parity status of every function is pinned by ``tests/test_oracle_*.py``
(closed forms, brute force, identities, finite differences, the worked
example); the tolerance tensors by ``tests/test_oracle_tolerance.py`` (an
independent model of the kernels' arithmetic lands inside them, planted
mistakes land outside); the bias statistics of ``bias.py`` by
``tests/test_bias_stats.py``.  Nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

RNE, RNA, RTZ, RD, RU = 0, 1, 2, 3, 4
MODES = {"rne": RNE, "rna": RNA, "rtz": RTZ, "rd": RD, "ru": RU}

_P = ctypes.c_void_p


class _Problem(ctypes.Structure):
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("dO", _P),
                ("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("D", ctypes.c_int),
                ("scale", ctypes.c_double), ("causal", ctypes.c_int), ("stabilise", ctypes.c_int),
                ("beta", ctypes.c_double)]


_FWD_FIELDS = ["O", "O_stab", "tol_O", "lse", "tol_lse", "rowmax", "shift", "pbar_max",
               "ties", "pbar_one", "near_ones", "amb_tie", "amb_pbar", "amb_near", "flags"]
_FWD_INT = {"ties", "pbar_one", "near_ones", "amb_tie", "amb_pbar", "amb_near", "flags"}
_FWD_ROWWISE = {"O", "O_stab", "tol_O"}


class _FwdOut(ctypes.Structure):
    _fields_ = [(f, _P) for f in _FWD_FIELDS]


_BWD_FIELDS = ["delta", "tol_delta", "dQ", "dK", "dV", "tol_dQ", "tol_dK", "tol_dV"]


class _BwdOut(ctypes.Structure):
    _fields_ = [(f, _P) for f in _BWD_FIELDS]


_lib = None


def lib():
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        L.orc_bf16_decode.restype = ctypes.c_double
        L.orc_bf16_decode.argtypes = [ctypes.c_uint16]
        L.orc_bf16_round2.restype = ctypes.c_uint16
        L.orc_bf16_round2.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int]
        L.orc_bf16_from_double.restype = ctypes.c_uint16
        L.orc_bf16_from_double.argtypes = [ctypes.c_double, ctypes.c_int]
        L.orc_bf16_add.restype = ctypes.c_uint16
        L.orc_bf16_add.argtypes = [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_int]
        L.orc_bf16_round_array.restype = None
        L.orc_bf16_round_array.argtypes = [_P, ctypes.c_int64, ctypes.c_int, _P]
        L.orc_exact_dot.restype = ctypes.c_int
        L.orc_exact_dot.argtypes = [_P, _P, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
        L.orc_shift_rule.restype = ctypes.c_double
        L.orc_shift_rule.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        L.orc_forward.restype = ctypes.c_int
        L.orc_forward.argtypes = [ctypes.POINTER(_Problem), _P, ctypes.c_int64, ctypes.POINTER(_FwdOut)]
        L.orc_backward.restype = ctypes.c_int
        L.orc_backward.argtypes = [ctypes.POINTER(_Problem), _P, ctypes.c_int64, _P, _P, _P, _P,
                                   ctypes.POINTER(_BwdOut)]
        L.orc_emulate_pv.restype = ctypes.c_int
        L.orc_emulate_pv.argtypes = [ctypes.POINTER(_Problem), _P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _P, _P]
        L.orc_online_ones.restype = ctypes.c_int
        L.orc_online_ones.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, _P, ctypes.c_int64, _P, _P]
        L.orc_threads.restype = ctypes.c_int
        L.orc_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16), got %s" % a.dtype)
    return a


# ---------------------------------------------------------------- soft-float

def bf16_decode(bits) -> np.ndarray:
    """Exact value of each bf16 bit pattern, as float64."""
    b = np.asarray(bits, dtype=np.uint16)
    f = lib().orc_bf16_decode
    return np.array([f(int(x)) for x in b.ravel()], dtype=np.float64).reshape(b.shape)


def bf16_from_double(x, mode: str = "rne") -> np.ndarray:
    """Correctly rounded bf16 bits of float64 values in the given rounding mode."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_bf16_round_array(_ptr(a), a.size, MODES[mode], _ptr(out))
    return out


def bf16_round2(hi: float, lo: float, mode: str = "rne") -> int:
    """bf16 bits of the exact value hi + lo (|lo| at most half an ulp of hi)."""
    return int(lib().orc_bf16_round2(float(hi), float(lo), MODES[mode]))


def bf16_add(a: int, b: int, mode: str = "rne") -> int:
    """bf16 bits of the exact sum of two bf16 values, rounded once."""
    return int(lib().orc_bf16_add(int(a), int(b), MODES[mode]))


def exact_dot(a_bits, b_bits):
    """(value, certified_fast_path) of the exact dot product of two bf16 vectors."""
    a = _bits(a_bits)
    b = _bits(b_bits)
    v = ctypes.c_double()
    fast = lib().orc_exact_dot(_ptr(a), _ptr(b), a.size, ctypes.byref(v))
    return v.value, bool(fast)


def shift_rule(rm: float, rs: int, stabilise: bool, beta: float) -> float:
    """m* of the duplicate-max rule, in scaled score units."""
    return float(lib().orc_shift_rule(float(rm), int(rs), int(bool(stabilise)), float(beta)))


def threads() -> int:
    """OpenMP threads the last oracle call ran on."""
    return int(lib().orc_threads())


# ---------------------------------------------------------------- attention

def _problem(q, k, v, dO, scale, causal, stabilise, beta):
    q = _bits(q)
    k = _bits(k)
    v = None if v is None else _bits(v)
    dO = None if dO is None else _bits(dO)
    if q.ndim != 4 or k.shape != q.shape or (v is not None and v.shape != q.shape) or \
            (dO is not None and dO.shape != q.shape):
        raise ValueError("q, k, v, dO must share one [B, H, N, D] shape")
    B, H, N, D = q.shape
    p = _Problem(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), B, H, N, D, float(scale), int(bool(causal)),
                 int(bool(stabilise)), float(beta))
    return p, (q, k, v, dO), (B, H, N, D)


def forward(q, k, v=None, *, scale: float, causal: bool, stabilise: bool = False, beta: float = 2.0,
            rows: Optional[Sequence[int]] = None, want: Optional[Sequence[str]] = None) -> dict:
    """Oracle forward over every row (or the flattened rows given).

    Returns a dict of numpy arrays shaped [B, H, N] (or [B, H, N, D]) holding the
    fields in ``want`` (default: all; rows not computed are NaN / -1).
    """
    p, keep, (B, H, N, D) = _problem(q, k, v, None, scale, causal, stabilise, beta)
    want = list(_FWD_FIELDS if want is None else want)
    if v is None:
        want = [w for w in want if w not in _FWD_ROWWISE]
    res = {}
    out = _FwdOut()
    for f in want:
        shape = (B, H, N, D) if f in _FWD_ROWWISE else (B, H, N)
        arr = np.full(shape, -1, dtype=np.int32) if f in _FWD_INT else np.full(shape, np.nan)
        res[f] = arr
        setattr(out, f, _ptr(arr))
    rr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    rc = lib().orc_forward(ctypes.byref(p), _ptr(rr), 0 if rr is None else rr.size, ctypes.byref(out))
    if rc != 0:
        raise ValueError("oracle forward rejected the inputs (non-finite values)")
    return res


def backward(q, k, v, dO, fwd: dict, *, scale: float, causal: bool,
             heads: Optional[Sequence[int]] = None) -> dict:
    """Oracle backward for every head (or the flattened heads b*H + h given).

    ``fwd`` must hold O, tol_O, lse and tol_lse from :func:`forward` for every
    row of those heads.
    """
    p, keep, (B, H, N, D) = _problem(q, k, v, dO, scale, causal, False, 2.0)
    res = {}
    out = _BwdOut()
    for f in _BWD_FIELDS:
        shape = (B, H, N) if f in ("delta", "tol_delta") else (B, H, N, D)
        arr = np.full(shape, np.nan)
        res[f] = arr
        setattr(out, f, _ptr(arr))
    hh = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    O = np.ascontiguousarray(fwd["O"], dtype=np.float64)
    tO = np.ascontiguousarray(fwd["tol_O"], dtype=np.float64)
    lse = np.ascontiguousarray(fwd["lse"], dtype=np.float64)
    tl = np.ascontiguousarray(fwd["tol_lse"], dtype=np.float64)
    rc = lib().orc_backward(ctypes.byref(p), _ptr(hh), 0 if hh is None else hh.size, _ptr(O),
                            _ptr(lse), _ptr(tO), _ptr(tl), ctypes.byref(out))
    if rc != 0:
        raise ValueError("oracle backward rejected the inputs")
    return res


def emulate_bf16_pv(q, k, v, *, scale: float, causal: bool, stabilise: bool = False, beta: float = 2.0,
                    accumulate: str = "rne", round_pbar: bool = True,
                    rows: Optional[Sequence[int]] = None) -> dict:
    """P_bar V accumulated in bf16, one rounding per product and per addition
    (see ``emulate_row`` in oracle.c), normalised by the FP64 row sum.

    accumulate: a rounding mode ("rne", "rna", "rtz", "rd", "ru") or "exact"
    (FP64 accumulation of the exact products).  Returns {"O": [B, H, N, D]
    float64, "events": [B, H, N] int32 = P_bar entries equal to 1}; rows not
    computed are NaN / -1.
    """
    p, keep, (B, H, N, D) = _problem(q, k, v, None, scale, causal, stabilise, beta)
    O = np.full((B, H, N, D), np.nan)
    ev = np.full((B, H, N), -1, dtype=np.int32)
    rr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    mode = -1 if accumulate == "exact" else MODES[accumulate]
    rc = lib().orc_emulate_pv(ctypes.byref(p), _ptr(rr), 0 if rr is None else rr.size, int(bool(round_pbar)),
                              mode, _ptr(O), _ptr(ev))
    if rc != 0:
        raise ValueError("oracle emulation rejected the inputs")
    return {"O": O, "events": ev}


def online_ones(q, k, *, scale: float, causal: bool, stabilise: bool, beta: float = 2.0, tile: int = 64,
                rows: Optional[Sequence[int]] = None) -> dict:
    """Keys per row whose P_bar rounds to a bf16 1.0 when the duplicate-max rule
    is applied online: the running (max, count) merged tile by tile in key
    order (tiles of ``tile`` keys from key 0) and each tile's P_bar formed
    with the shift of the pair after that tile (``online_row`` in oracle.c).

    Returns {"ones": [B, H, N] int32, "amb": [B, H, N] int32}; rows not
    computed are -1.
    """
    p, keep, (B, H, N, D) = _problem(q, k, None, None, scale, causal, stabilise, beta)
    ones = np.full((B, H, N), -1, dtype=np.int32)
    amb = np.full((B, H, N), -1, dtype=np.int32)
    rr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    rc = lib().orc_online_ones(ctypes.byref(p), int(tile), _ptr(rr), 0 if rr is None else rr.size, _ptr(ones),
                               _ptr(amb))
    if rc != 0:
        raise ValueError("oracle online count rejected the inputs")
    return {"ones": ones, "amb": amb}


def head_rows(heads: Sequence[int], N: int) -> np.ndarray:
    """Flattened row indices of every row of the given flattened heads."""
    h = np.asarray(heads, dtype=np.int64)
    return (h[:, None] * N + np.arange(N, dtype=np.int64)[None, :]).ravel()
