"""The C-ABI library loads and exports every symbol of include/fa.h; host-side validation and
error behaviour (CPU only: no call here reaches a HIP API)."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in ("fa_fwd", "fa_fwd_o32", "fa_decode", "fa_decode_workspace_size",
                 "fa_validate_fwd", "fa_validate_decode", "fa_status_str", "fa_last_hip_error"):
        assert name in fns


def test_every_declared_symbol_is_exported(fa_lib):
    exported = subprocess.run(["nm", "-D", "--defined-only", fa_lib.LIB_PATH], capture_output=True,
                              text=True, check=True).stdout
    syms = set(re.findall(r"\sT\s+(\w+)$", exported, flags=re.M))
    for name in header_functions():
        assert name in syms, f"{name} declared in fa.h but not exported"
        assert getattr(ctypes.CDLL(fa_lib.LIB_PATH), name)


def test_binding_covers_every_declared_function(fa_lib):
    from io_aware_attention_fa_amd import _lib
    assert sorted(_lib.SIGNATURES) == header_functions()
    for name in header_functions():
        assert callable(getattr(fa_lib, name))


def test_status_strings(fa_lib):
    seen = set()
    for code in range(0, 12):
        s = fa_lib.fa_status_str(code)
        assert s and s not in seen
        seen.add(s)
    assert "unknown" in fa_lib.fa_status_str(12345)
    assert fa_lib.fa_last_hip_error() == 0


P = 0x100000   # a 16-byte aligned fake address; validation never dereferences pointers


@pytest.mark.parametrize("args,code", [
    ((P, P, P, P, P, 1, 1, 16, 16, 64, 0, 0.125), 0),
    ((0, P, P, P, P, 1, 1, 16, 16, 64, 0, 0.125), 1),
    ((P, P, P, P, 0, 1, 1, 16, 16, 64, 0, 0.125), 1),
    ((P, P, P, P, P, 0, 1, 16, 16, 64, 0, 0.125), 2),
    ((P, P, P, P, P, 1, -1, 16, 16, 64, 0, 0.125), 2),
    ((P, P, P, P, P, 1, 1, 0, 16, 64, 0, 0.125), 2),
    ((P, P, P, P, P, 1, 1, 16, 0, 64, 0, 0.125), 2),
    ((P, P, P, P, P, 1, 1, 16, 2**30, 128, 0, 0.125), 2),
    ((P, P, P, P, P, 1, 1, 16, 16, 100, 0, 0.125), 3),
    ((P, P, P, P, P, 1, 1, 16, 16, 136, 0, 0.125), 3),
    ((P, P, P, P, P, 1, 1, 16, 16, 256, 0, 0.125), 3),
    ((P, P, P, P, P, 1, 1, 16, 16, 4, 0, 0.125), 3),
    ((P, P, P, P, P, 1, 1, 16, 16, 96, 0, 0.125), 0),
    ((P, P, P, P, P, 1, 1, 16, 16, 80, 0, 0.125), 0),
    ((P, P, P, P, P, 1, 1, 16, 16, 8, 0, 0.125), 0),
    ((P, P, P, P, P, 1, 1, 17, 16, 64, 1, 0.125), 4),
    ((P, P, P, P, P, 1, 1, 16, 17, 64, 1, 0.125), 0),
    ((P, P, P, P, P, 1, 1, 17, 16, 64, 0, 0.125), 0),
    ((P + 8, P, P, P, P, 1, 1, 16, 16, 64, 0, 0.125), 5),
    ((P, P, P, P, P + 2, 1, 1, 16, 16, 64, 0, 0.125), 5),
    ((P, P, P, P, P, 1, 1, 16, 16, 64, 0, math.inf), 6),
    ((P, P, P, P, P, 1, 1, 16, 16, 64, 0, math.nan), 6),
    ((P, P, P, P, P, 1, 1, 16, 16, 64, 2, 0.125), 6),
])
def test_validate_fwd(fa_lib, args, code):
    assert fa_lib.fa_validate_fwd(*args) == code


@pytest.mark.parametrize("B,h,Tk,d,S,ws_delta,code", [
    (2, 3, 100, 128, 4, 0, 0),
    (2, 3, 100, 128, 0, 0, 7),
    (2, 3, 100, 128, 101, 0, 7),
    (2, 3, 300, 128, 257, 0, 7),
    (2, 3, 100, 128, 100, 0, 0),
    (2, 3, 100, 128, 4, -4, 8),
    (2, 3, 100, 80, 4, 0, 0),      # padded head dims run the padded kernels
    (2, 3, 100, 8, 4, 0, 0),
    (2, 3, 100, 84, 4, 0, 3),      # not a multiple of 8
    (2, 3, 100, 136, 4, 0, 3),     # above 128
    (0, 3, 100, 128, 4, 0, 2),
])
def test_validate_decode(fa_lib, B, h, Tk, d, S, ws_delta, code):
    ws = max(fa_lib.fa_decode_workspace_size(max(B, 1), h, d, max(S, 1)) + ws_delta, 0)
    assert fa_lib.fa_validate_decode(P, P, P, P, P, B, h, Tk, d, 0.1, S, P, ws) == code


def test_decode_workspace_size(fa_lib):
    assert fa_lib.fa_decode_workspace_size(64, 32, 128, 16) == 64 * 32 * 16 * 130 * 4
    assert fa_lib.fa_decode_workspace_size(0, 32, 128, 16) == 0
    # other head dims are computed at the padded width (64 or 128)
    assert fa_lib.fa_decode_workspace_size(2, 3, 80, 4) == 2 * 3 * 4 * 130 * 4
    assert fa_lib.fa_decode_workspace_size(2, 3, 8, 4) == 2 * 3 * 4 * 66 * 4
    assert fa_lib.fa_validate_decode(P, P, P, P, P, 1, 1, 10, 64, 0.1, 2, 0, 10**6) == 8
    assert fa_lib.fa_validate_decode(P, P, P, P, P, 1, 1, 10, 64, 0.1, 2, P + 4, 10**6) == 8


def test_invalid_calls_touch_nothing(fa_lib):
    """Entry points return the validation code before any HIP call; outputs stay untouched.

    Host arrays stand in for device buffers: a rejected call never dereferences them.
    """
    from io_aware_attention_fa_amd import _lib
    buf = np.zeros(4096, dtype=np.uint16)
    o = np.full(4096, 0x7FC1, dtype=np.uint16)
    lse = np.full(64, 12345.0, dtype=np.float32)
    ws = np.full(4096, 7, dtype=np.uint8)
    a = [ctypes.c_void_p(x.ctypes.data) for x in (buf, buf, buf, o, lse)]
    st = _lib.lib.fa_fwd(*a, 1, 1, 16, 16, 100, 0, 0.125, None)
    assert st == 3
    st = _lib.lib.fa_fwd_o32(*a, 1, 1, 17, 16, 64, 1, 0.125, None)
    assert st == 4
    st = _lib.lib.fa_decode(*a, 1, 1, 16, 64, 0.125, 17, ctypes.c_void_p(ws.ctypes.data),
                            ws.nbytes, None)
    assert st == 7
    assert np.all(o == 0x7FC1) and np.all(lse == 12345.0) and np.all(ws == 7)


def test_bwd_workspace_size(fa_lib):
    # two fp32 arrays of B*h*Tq values, each rounded up to 256 bytes, then 1 KB of item counters
    n = 2 * 3 * 100 * 4
    assert fa_lib.fa_bwd_workspace_size(2, 3, 100) == 2 * ((n + 255) // 256 * 256) + 1024
    assert fa_lib.fa_bwd_workspace_size(0, 3, 100) == 0
    assert fa_lib.fa_bwd_workspace_size(1, 1, 64) == 512 + 1024


def _vb(fa_lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, h=2, Tq=100, Tk=120, d=128,
             causal=1, scale=0.1, ws=P, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = fa_lib.fa_bwd_workspace_size(max(a["B"], 1), max(a["h"], 1),
                                                     max(a["Tq"], 1))
    return fa_lib.fa_validate_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                  a["dk"], a["dv"], a["B"], a["h"], a["Tq"], a["Tk"], a["d"],
                                  a["causal"], a["scale"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    ({"do": 0}, 1), ({"dv": 0}, 1), ({"lse": 0}, 1),
    ({"Tq": 0}, 2), ({"B": 0}, 2), ({"Tk": 2**30}, 2),
    ({"d": 80}, 0), ({"d": 8}, 0), ({"d": 84}, 3), ({"d": 0}, 3), ({"d": 136}, 3),
    ({"Tq": 121}, 4), ({"Tq": 121, "causal": 0}, 0),
    ({"do": P + 8}, 5), ({"dk": P + 2}, 5), ({"lse": P + 2}, 5),
    ({"scale": math.nan}, 6), ({"causal": 3}, 6),
    ({"ws": 0}, 8), ({"ws": P + 4}, 8), ({"ws_bytes": 100}, 8),
])
def test_validate_bwd(fa_lib, kw, code):
    assert _vb(fa_lib, **kw) == code


def test_invalid_bwd_call_touches_nothing(fa_lib):
    from io_aware_attention_fa_amd import _lib
    buf = np.zeros(4096, dtype=np.uint16)
    out = np.full(4096, 0x7FC1, dtype=np.uint16)
    lse = np.zeros(64, dtype=np.float32)
    ws = np.full(4096, 7, dtype=np.uint8)
    a = [ctypes.c_void_p(x.ctypes.data) for x in (buf, buf, buf, buf, buf, lse, out, out, out)]
    st = _lib.lib.fa_bwd(*a, 1, 1, 16, 16, 100, 0, 0.125, ctypes.c_void_p(ws.ctypes.data),
                         ws.nbytes, None)
    assert st == 3
    # fp32 outputs: unpadded head dims only
    st = _lib.lib.fa_bwd_f32(*a, 1, 1, 16, 16, 96, 0, 0.125, ctypes.c_void_p(ws.ctypes.data),
                             ws.nbytes, None)
    assert st == 3
    st = _lib.lib.fa_bwd_f32(*a, 1, 1, 17, 16, 64, 1, 0.125, ctypes.c_void_p(ws.ctypes.data),
                             ws.nbytes, None)
    assert st == 4
    assert np.all(out == 0x7FC1) and np.all(ws == 7)


@pytest.mark.parametrize("args,code", [
    ((P, P, 0, 4, 4096), 0), ((P, P, P, 4, 4096), 0),
    ((0, P, 0, 4, 4096), 1), ((P, 0, 0, 4, 4096), 1),
    ((P, P, 0, 0, 4096), 2), ((P, P, 0, 4, 0), 2), ((P, P, 0, 4, 2**31), 2),
    ((P + 2, P, 0, 4, 4096), 5), ((P, P, P + 1, 4, 4096), 5), ((P + 4, P + 8, 0, 3, 7), 0),
])
def test_validate_softmax(fa_lib, args, code):
    assert fa_lib.fa_validate_softmax(*args) == code


def test_invalid_softmax_call_touches_nothing(fa_lib):
    from io_aware_attention_fa_amd import _lib
    x = np.zeros(64, dtype=np.float32)
    y = np.full(64, 7.0, dtype=np.float32)
    st = _lib.lib.fa_softmax_rows(ctypes.c_void_p(x.ctypes.data), ctypes.c_void_p(y.ctypes.data),
                                  None, 0, 64, None)
    assert st == 2 and np.all(y == 7.0)


@pytest.mark.parametrize("args,code", [
    ((P, P, 1), 0), ((P, P, 2**40), 0), ((0, P, 5), 1), ((P, 0, 5), 1), ((P, P, 0), 2),
    ((P + 4, P, 5), 5), ((P, P + 8, 5), 5),
])
def test_validate_gelu(fa_lib, args, code):
    assert fa_lib.fa_validate_gelu(*args) == code


@pytest.mark.parametrize("args,code", [
    ((P, P, P, 4096, 8192, 0.1), 0), ((P, P, P, 3, 7, 0.0), 0), ((P + 2, P, P + 2, 3, 7, 0.5), 0),
    ((0, P, P, 4, 4, 0.1), 1), ((P, 0, P, 4, 4, 0.1), 1),
    ((P, P, P, 0, 4, 0.1), 2), ((P, P, P, 4, 0, 0.1), 2), ((P, P, P, 2**40, 2**40, 0.1), 2),
    ((P + 1, P, P, 4, 4, 0.1), 5),
    ((P, P, P, 4, 4, 1.0), 10), ((P, P, P, 4, 4, -0.1), 10), ((P, P, P, 4, 4, math.nan), 10),
])
def test_validate_bias_gelu_dropout(fa_lib, args, code):
    assert fa_lib.fa_validate_bias_gelu_dropout(*args) == code


def _vs(fa_lib, **kw):
    a = dict(B=2, h=3, Tq=100, Tk=120, d=80, causal=1, scale=0.1,
             qs=(3 * 100 * 80, 100 * 80, 80), ks=(120 * 3 * 80, 80, 3 * 80),
             vs=(120 * 3 * 80, 80, 3 * 80), os=(3 * 100 * 80, 100 * 80, 80))
    a.update(kw)
    return fa_lib.fa_validate_fwd_strided(P, P, P, P, P, a["B"], a["h"], a["Tq"], a["Tk"], a["d"],
                                          a["qs"], a["ks"], a["vs"], a["os"], a["causal"],
                                          a["scale"])


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    # broadcast inputs (one q, k, v head for every batch and head) are fine ...
    ({"d": 128, "qs": (0, 0, 128), "ks": (0, 0, 128), "vs": (0, 0, 128),
      "os": (3 * 100 * 128, 100 * 128, 128)}, 0),
    # ... a broadcast or self-overlapping output is not: several workgroups would write one element
    ({"d": 128, "qs": (0, 0, 128), "ks": (0, 0, 128), "vs": (0, 0, 128), "os": (0, 0, 128)}, 2),
    ({"os": (0, 100 * 80, 80)}, 2),                  # batches share the output
    ({"os": (3 * 100 * 80, 50 * 80, 80)}, 2),        # heads overlap by 50 rows
    ({"os": (3 * 100 * 80, 100 * 80, 40)}, 2),       # row stride below d is caught as well
    ({"os": (100 * 3 * 80, 80, 3 * 80)}, 0),         # [B][T][h][d] output
    ({"os": (80, 2 * 100 * 80, 2 * 80)}, 0),         # [h][T][B][d] output: interleaved, no overlap
    ({"os": (80, 100 * 80, 80)}, 2),                 # batch stride inside a row's span
    ({"qs": None}, 2),
    ({"ks": (120 * 3 * 80, 80, 72)}, 2),            # row stride below d
    ({"ks": (120 * 3 * 80, 80, 3 * 80 + 4)}, 2),    # row stride not a multiple of 8
    ({"vs": (120 * 3 * 80, 84, 3 * 80)}, 2),        # head stride not a multiple of 8
    ({"os": (-8, 100 * 80, 80)}, 2),                # negative stride
    ({"ks": (0, 0, 2**26)}, 2),                      # head beyond 2^31 bytes
    ({"d": 100}, 3), ({"Tq": 121, "os": (3 * 121 * 80, 121 * 80, 80)}, 4),
])
def test_validate_fwd_strided(fa_lib, kw, code):
    assert _vs(fa_lib, **kw) == code


def _vbs(fa_lib, **kw):
    qs = (3 * 100 * 80, 80, 3 * 80)   # [B][T][h][d] storage of q, o, do, dq
    ks = (3 * 120 * 80, 80, 3 * 80)   # ... of k, v, dk, dv
    a = dict(B=2, h=3, Tq=100, Tk=120, d=80, causal=1, scale=0.1, ws=P, ws_bytes=None,
             strides=[qs, ks, ks, qs, qs, qs, ks, ks], lse=P, dk=P)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = fa_lib.fa_bwd_workspace_size(2, 3, 100)
    return fa_lib.fa_validate_bwd_strided(P, P, P, P, P, a["lse"], P, a["dk"], P, a["B"], a["h"],
                                          a["Tq"], a["Tk"], a["d"], a["strides"], a["causal"],
                                          a["scale"], a["ws"], a["ws_bytes"])


_QS, _KS = (3 * 100 * 80, 80, 3 * 80), (3 * 120 * 80, 80, 3 * 80)


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    ({"d": 64, "strides": [(0, 0, 64)] * 5 + [(3 * 100 * 64, 100 * 64, 64)] +
      [(3 * 120 * 64, 120 * 64, 64)] * 2}, 0),       # broadcast inputs, distinct gradients
    ({"d": 8, "strides": [(0, 0, 8)] * 5 + [_QS, _KS, _KS]}, 0),
    # a broadcast or self-overlapping gradient tensor is rejected
    ({"d": 64, "strides": [(0, 0, 64)] * 8}, 2),
    ({"strides": [_QS, _KS, _KS, _QS, _QS, (0, 80, 3 * 80), _KS, _KS]}, 2),     # dq batches alias
    ({"strides": [_QS, _KS, _KS, _QS, _QS, _QS, (3 * 120 * 80, 0, 3 * 80), _KS]}, 2),  # dk heads
    ({"strides": [_QS, _KS, _KS, _QS, _QS, _QS, _KS, (3 * 120 * 80, 80, 80)]}, 2),   # dv rows
    # packed gradients ([B][T][3][h][d], dq/dk/dv interleaved) do not alias themselves
    ({"Tk": 100, "strides": [_QS] * 5 + [(300 * 3 * 80, 80, 9 * 80)] * 3}, 0),
    ({"lse": 0}, 1), ({"dk": 0}, 1),
    ({"strides": [_QS, _KS, _KS, _QS, _QS, _QS, _KS, None]}, 2),
    ({"strides": [_QS, _KS, _KS, _QS, (3 * 100 * 80, 80, 72), _QS, _KS, _KS]}, 2),   # do row < d
    ({"strides": [_QS, _KS, _KS, _QS, _QS, _QS, (3 * 120 * 80, 84, 3 * 80), _KS]}, 2),
    ({"strides": [_QS, (0, 0, 2**26), _KS, _QS, _QS, _QS, _KS, _KS]}, 2),   # k head > 2^31 B
    ({"d": 100}, 3), ({"d": 136}, 3),
    ({"Tq": 121, "strides": [_QS, _KS, _KS, _QS, _QS, (3 * 121 * 80, 80, 3 * 80), _KS, _KS]}, 4),
    ({"lse": P + 2}, 5), ({"dk": P + 8}, 5),
    ({"causal": 2}, 6), ({"ws_bytes": 16}, 8),
])
def test_validate_bwd_strided(fa_lib, kw, code):
    assert _vbs(fa_lib, **kw) == code


def test_invalid_bwd_strided_call_touches_nothing(fa_lib):
    from io_aware_attention_fa_amd import _lib
    buf = np.zeros(4096, dtype=np.uint16)
    out = np.full(4096, 0x7FC1, dtype=np.uint16)
    lse = np.zeros(64, dtype=np.float32)
    ws = np.full(4096, 7, dtype=np.uint8)
    a = [ctypes.c_void_p(x.ctypes.data) for x in (buf, buf, buf, buf, buf, lse, out, out, out)]
    s3 = (ctypes.c_int64 * 3)(16 * 104, 104, 104)
    st = _lib.lib.fa_bwd_strided(*a, 1, 1, 16, 16, 100, *([s3] * 8), 0, 0.125,
                                 ctypes.c_void_p(ws.ctypes.data), ws.nbytes, None)
    assert st == 3
    assert np.all(out == 0x7FC1) and np.all(ws == 7)



def _vds(fa_lib, **kw):
    a = dict(B=2, h=3, Tk=500, d=80, qs=(3 * 80, 80), ks=(500 * 3 * 80, 80, 3 * 80),
             vs=(500 * 3 * 80, 80, 3 * 80), os=(3 * 80, 80), scale=0.1, S=4, ws=P, ws_bytes=None,
             o=P, q=P)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = fa_lib.fa_decode_workspace_size(2, 3, a["d"], 4)
    return fa_lib.fa_validate_decode_strided(a["q"], P, P, a["o"], P, a["B"], a["h"], a["Tk"],
                                             a["d"], a["qs"], a["ks"], a["vs"], a["os"],
                                             a["scale"], a["S"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    ({"d": 128, "qs": (0, 128), "ks": (0, 0, 128), "vs": (0, 0, 128), "os": (3 * 128, 128)}, 0),
    ({"d": 128, "qs": (0, 128), "ks": (0, 0, 128), "vs": (0, 0, 128), "os": (0, 128)}, 2),
    ({"os": (80, 80)}, 2), ({"os": (3 * 80, 40)}, 2),   # output rows alias
    ({"os": (80, 2 * 80)}, 0),                          # [h][B][d] output
    ({"o": P + 2}, 0),                       # o needs only 2-byte alignment
    ({"o": 0}, 1),
    ({"qs": None}, 2), ({"os": (3 * 80, 84)}, 2), ({"ks": (500 * 3 * 80, 80, 72)}, 2),
    ({"vs": (0, 0, 2**25)}, 2),              # (Tk + 256) rows beyond 2^31 bytes
    ({"d": 100}, 3), ({"d": 136}, 3),
    ({"q": P + 8}, 5), ({"o": P + 1}, 5),
    ({"scale": math.inf}, 6), ({"S": 0}, 7), ({"S": 501}, 7), ({"ws_bytes": 64}, 8),
])
def test_validate_decode_strided(fa_lib, kw, code):
    assert _vds(fa_lib, **kw) == code


def test_noalloc_decode_rejects_before_any_hip_call(fa_lib):
    """fa_decode_noalloc: argument errors and partials beyond the static array are reported before
    the library touches the GPU, with every output untouched."""
    from io_aware_attention_fa_amd import _lib
    buf = np.zeros(64, dtype=np.uint16)
    out = np.full(64, 0x7FC1, dtype=np.uint16)
    lse = np.full(4, 5.0, dtype=np.float32)
    a = [ctypes.c_void_p(x.ctypes.data) for x in (buf, buf, buf, out, lse)]
    call = lambda B, h, Tk, d, S: _lib.lib.fa_decode_noalloc(*a, B, h, Tk, d, 0.125, S, None)
    assert fa_lib.FA_NOALLOC_SCRATCH_BYTES == 32 * 2**20
    # B=64, h=32, d=128: 31 splits fit in the array, 32 do not
    assert fa_lib.fa_decode_workspace_size(64, 32, 128, 31) <= fa_lib.FA_NOALLOC_SCRATCH_BYTES
    assert call(64, 32, 8192, 128, 32) == fa_lib.FA_ERR_SCRATCH
    assert call(1, 1, 300, 128, 0) == fa_lib.FA_ERR_SPLITS
    assert call(1, 1, 300, 100, 4) == fa_lib.FA_ERR_HEAD_DIM
    assert _lib.lib.fa_decode_noalloc(None, *a[1:], 1, 1, 300, 128, 0.125, 4, None) == 1
    assert np.all(out == 0x7FC1) and np.all(lse == 5.0)
    assert "FA_NOALLOC_SCRATCH_BYTES" in fa_lib.fa_status_str(fa_lib.FA_ERR_SCRATCH)
