"""The C ABI without a GPU: the library loads, exports every function that
include/attn.h declares, and rejects each invalid argument before any HIP
call.  Every call here fails validation, so no kernel is launched and the
fake (never dereferenced) device addresses are never used."""
import ctypes
import math
import os
import subprocess

import pytest

from numerics_safe_softmax_amd import binding

LIB = binding.LIB_PATH
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libattn.so not built")

A = 0x10000          # fake, 16-byte aligned addresses (validation rejects before use)
STEP = 0x10000000    # far apart: no overlaps


def addr(i):
    return A + i * STEP


def lib():
    return binding.lib()


def test_exports_every_header_function():
    names = binding.header_functions()
    assert set(names) >= {"attn_fwd", "attn_bwd", "attn_tiecount", "attn_status_string", "attn_fwd_o32",
                          "attn_bwd_o32", "attn_bwd_dq", "attn_bwd_dkdv", "attn_abi_version",
                          "attn_fwd_key_tile"}
    L = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10):
        assert binding.status_string(s) and binding.status_string(s) != "unknown attn_status"
    assert binding.status_string(12345) == "unknown attn_status"
    # the shape status names the limits the check enforces (N and the launch grid)
    shape_text = binding.status_string(-2)
    assert "2^24" in shape_text and "ceil(N/128)" in shape_text and "2^31" not in shape_text
    assert binding.abi_version() == 5


def test_forward_key_tile():
    # a pure query (no device call): the forward's KV tile width per head size
    assert binding.fwd_key_tile(64) == 64
    assert binding.fwd_key_tile(128) == 32
    for D in (0, 32, 96, 256, -64):
        assert lib().attn_fwd_key_tile(D) == -3
        with pytest.raises(binding.AttnError):
            binding.fwd_key_tile(D)


def fwd(**kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), o=addr(3), lse=addr(4), ties=None, pone=None, formed=None,
             B=1, H=2, N=64, D=64, scale=0.125, causal=1, stab=1, beta=2.0)
    a.update(kw)
    return lib().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ties"], a["pone"], a["formed"],
                          a["B"], a["H"], a["N"], a["D"], a["scale"], a["causal"], a["stab"], a["beta"], None)


def bwd(**kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), o=addr(3), dO=addr(4), lse=addr(5), dq=addr(6), dk=addr(7),
             dv=addr(8), delta=addr(9), ws=addr(10), wsb=1 << 40, B=1, H=2, N=64, D=64, scale=0.125, causal=1,
             stab=1, beta=2.0)
    a.update(kw)
    return lib().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["dO"], a["lse"], a["dq"], a["dk"], a["dv"],
                          a["delta"], a["ws"], a["wsb"], a["B"], a["H"], a["N"], a["D"], a["scale"], a["causal"],
                          a["stab"], a["beta"], None)


def tie(**kw):
    a = dict(q=addr(0), k=addr(1), ties=addr(2), rowmax=None, B=1, H=2, N=64, D=64, scale=0.125, causal=1)
    a.update(kw)
    return lib().attn_tiecount(a["q"], a["k"], a["ties"], a["rowmax"], a["B"], a["H"], a["N"], a["D"],
                               a["scale"], a["causal"], None)


@pytest.mark.parametrize("call", [fwd, bwd])
def test_forward_and_backward_validation(call):
    assert call(q=None) == -1
    assert call(B=-1) == -2
    assert call(N=-5) == -2
    assert call(B=1 << 14, H=1 << 14, N=1 << 10) == -2
    assert call(N=1 << 24) == -2                       # row indices stay 32-bit
    assert call(B=1 << 12, H=1 << 12, N=1) == -2       # 2^24 workgroups
    assert call(B=1 << 10, H=1 << 10, N=2048) == -2    # 2^20 heads x 16 row tiles
    # 2^31 elements per tensor is a valid shape: the call gets past the shape
    # check and stops at the (fake, 256 MB apart) addresses' overlap instead
    assert call(B=64, H=512, N=1024) == -7
    assert call(D=96) == -3
    assert call(D=32) == -3
    assert call(beta=1.0) == -4
    assert call(beta=float("nan")) == -4
    assert call(beta=math.inf) == -4
    assert call(scale=0.0) == -5
    assert call(scale=-1.0) == -5
    assert call(scale=float("inf")) == -5
    assert call(k=addr(1) + 8) == -6
    assert call(q=addr(0) + 2) == -6
    assert call(stab=3) == -10
    assert call(stab=-1) == -10


def test_beta_ignored_when_not_stabilised():
    # beta is only checked in stabilised mode; the call then proceeds to alias checks
    assert fwd(stab=0, beta=0.5, o=addr(0)) == -7


def test_alias_detection():
    assert fwd(o=addr(0)) == -7                  # o == q
    assert fwd(lse=addr(2) + 64) == -7           # lse inside v
    assert fwd(ties=addr(3) + 16) == -7          # ties inside o
    assert fwd(ties=addr(5), pone=addr(5)) == -7  # two outputs overlap
    assert bwd(dq=addr(4)) == -7                 # dq == dO
    assert bwd(delta=addr(6) + 32) == -7         # delta inside dq
    assert tie(ties=addr(1)) == -7


def test_empty_problems_return_ok_without_a_device():
    assert fwd(q=None, k=None, v=None, o=None, lse=None, B=0) == 0
    assert fwd(q=None, k=None, v=None, o=None, lse=None, N=0) == 0
    assert bwd(H=0, q=None) == 0
    assert tie(N=0, q=None) == 0


def test_tiecount_and_split_backward_validation():
    assert tie(ties=None) == -1
    assert tie(D=80) == -3
    assert tie(scale=math.nan) == -5
    L = lib()
    args = [addr(i) for i in range(8)] + [1, 2, 64, 64, 0.125, 1, None]
    bad = list(args)
    bad[6] = None
    assert L.attn_bwd_dq(*bad) == -1
    bad = list(args)
    bad[11] = 100
    assert L.attn_bwd_dkdv(*bad) == -3
    bad = list(args)
    bad[7] = addr(0)
    assert L.attn_bwd_dkdv(*bad) == -7


def test_fp32_o_entries_validation():
    L = lib()
    # attn_fwd_o32(q, k, v, o, o32, lse, ties, pone, formed, B, H, N, D, scale, causal, stab, beta, stream)
    base = [addr(0), addr(1), addr(2), addr(3), addr(4), addr(5), None, None, None, 1, 2, 64, 64, 0.125, 1, 1, 2.0,
            None]
    bad = list(base)
    bad[4] = None
    assert L.attn_fwd_o32(*bad) == -1          # o32 is required here
    bad = list(base)
    bad[4] = addr(4) + 4
    assert L.attn_fwd_o32(*bad) == -6
    bad = list(base)
    bad[4] = addr(2) + 64
    assert L.attn_fwd_o32(*bad) == -7          # o32 inside v
    bad = list(base)
    bad[15] = 5
    assert L.attn_fwd_o32(*bad) == -10
    bad = list(base)
    bad[5] = addr(4) + 4096
    assert L.attn_fwd_o32(*bad) == -7          # lse inside o32 (fp32: twice the bf16 bytes)
    # attn_bwd_o32(q, k, v, o32, dO, lse, dq, dk, dv, delta, ws, ws_bytes, B, H, N, D, scale, causal, stab,
    #              beta, stream)
    b = [addr(i) for i in range(11)] + [1 << 26, 1, 2, 64, 64, 0.125, 1, 1, 2.0, None]
    bad = list(b)
    bad[3] = None
    assert L.attn_bwd_o32(*bad) == -1
    bad = list(b)
    bad[6] = addr(3) + 16
    assert L.attn_bwd_o32(*bad) == -7          # dq inside o32
    bad = list(b)
    bad[15] = 80
    assert L.attn_bwd_o32(*bad) == -3
    bad = list(b)
    bad[10], bad[11] = None, 0
    assert L.attn_bwd_o32(*bad) == -9          # no workspace needed: stops at the device check
    assert L.attn_bwd_o32(*(b[:12] + [0] + b[13:])) == 0   # empty problem


def test_workspace_size_and_validation():
    L = lib()
    # the backward needs no workspace: 0 for every shape, valid or not
    for shape in ((2, 3, 100, 64), (2, 3, 100, 128), (0, 3, 100, 64), (1, 1, 64, 96), (-1, 1, 64, 64)):
        assert L.attn_bwd_workspace_bytes(*shape) == 0
    # NULL with 0 bytes, or any buffer, passes validation (stops at the device check here)
    assert bwd(ws=None, wsb=0) == -9
    assert bwd(D=128, ws=None, wsb=0) == -9
    assert bwd(ws=addr(10) + 8, wsb=4) == -9
