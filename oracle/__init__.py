"""CPU oracle for lossless BF16 sign+exponent coding — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it (``wc_oracle.c`` parses and writes the container with
code of its own).

Thin ctypes layer over ``wc_oracle.c`` (plain, single-threaded C loops; see
that file for the page citations of each step).  Inputs and outputs are
NumPy arrays of BF16 bit patterns (``uint16``), container bytes (``uint8``)
and fp32/fp64 GEMV results.

Parity: every function here is pinned by ``tests/test_oracle.py`` (golden
fixtures, exhaustive bit patterns, brute-force counts, closed forms and exact
GEMV cases); no function is parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

BYTESPLIT = 0
K15 = 1
RAW = 2
COMPACT = 1  # container flag: escape symbols only, positions implied by the code-15 marks

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_ERRORS = {-1: "bad argument", -2: "size limit", -3: "corrupt container"}


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what}: {_ERRORS.get(code, code)} ({code})")
        self.code = code


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile wc_oracle.c into a shared library with gcc (plain -O2)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
             src, "-o", tmp])
        os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    U64 = ctypes.c_uint64
    I = ctypes.c_int
    lib.orc_histogram.argtypes = [I, P, U64, P]
    lib.orc_dictionary.argtypes = [I, P, U64, P, P, P]
    lib.orc_container_size.argtypes = [I, U64, U64, P]
    lib.orc_container_size_flags.argtypes = [I, I, U64, U64, P]
    lib.orc_encode.argtypes = [I, P, U64, P, U64, P]
    lib.orc_encode_flags.argtypes = [I, I, P, U64, P, U64, P]
    lib.orc_header_flags.argtypes = [P, U64, P]
    lib.orc_header_info.argtypes = [P, U64, P, P, P, P, P, P]
    lib.orc_decode.argtypes = [P, U64, P, U64]
    lib.orc_gemv_f32.argtypes = [P, U64, U64, P, ctypes.c_uint32, P]
    lib.orc_gemv_f64.argtypes = [P, U64, U64, P, ctypes.c_uint32, P, P]
    lib.orc_bits_per_weight.argtypes = [P, U64, P, P]
    lib.orc_choose_layout.argtypes = [P, U64, P]
    for f in (lib.orc_histogram, lib.orc_dictionary, lib.orc_container_size,
              lib.orc_encode, lib.orc_header_info, lib.orc_decode,
              lib.orc_gemv_f32, lib.orc_gemv_f64, lib.orc_bits_per_weight,
              lib.orc_choose_layout, lib.orc_container_size_flags, lib.orc_encode_flags,
              lib.orc_header_flags):
        f.restype = I
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(_LIB_PATH)
    return _lib


def use_library(path: str | None):
    """Point this module at another build of the oracle (None = the default).
    Used only by the tests that plant a mistake in a copy of the oracle."""
    global _lib
    _lib = None if path is None else _bind(path)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(st: int, what: str):
    if st != 0:
        raise OracleError(st, what)


def _u16(w) -> np.ndarray:
    a = np.ascontiguousarray(w)
    if a.dtype != np.uint16:
        raise TypeError("weights must be BF16 bit patterns (uint16)")
    return a.reshape(-1)


def nsym(layout: int) -> int:
    return 512 if layout == K15 else 256


def histogram(layout: int, w) -> np.ndarray:
    a = _u16(w)
    counts = np.zeros(nsym(layout), dtype=np.uint64)
    _check(_load().orc_histogram(layout, _ptr(a), a.size, _ptr(counts)), "histogram")
    return counts


def dictionary(layout: int, counts: np.ndarray, n: int):
    c = np.zeros(512, dtype=np.uint64)
    c[: len(counts)] = counts
    d = np.zeros(16, dtype=np.uint16)
    nd = ctypes.c_int(0)
    ne = ctypes.c_uint64(0)
    _check(_load().orc_dictionary(layout, _ptr(c), n, _ptr(d), ctypes.byref(nd),
                                  ctypes.byref(ne)), "dictionary")
    return d, nd.value, ne.value


def container_size(layout: int, n: int, n_esc: int, flags: int = 0) -> int:
    t = ctypes.c_uint64(0)
    if flags:
        st = _load().orc_container_size_flags(layout, flags, n, n_esc, ctypes.byref(t))
    else:
        st = _load().orc_container_size(layout, n, n_esc, ctypes.byref(t))
    _check(st, "container_size")
    return t.value


def choose_layout(w) -> int:
    """The layout (BYTESPLIT, K15 or RAW) with the smallest container."""
    a = _u16(w)
    lay = ctypes.c_int(-1)
    _check(_load().orc_choose_layout(_ptr(a), a.size, ctypes.byref(lay)), "choose_layout")
    return lay.value


def encode(layout: int, w, flags: int = 0) -> np.ndarray:
    """The container of w; flags=COMPACT drops the escape-position stream."""
    a = _u16(w)
    n_esc = 0
    if layout != RAW:
        counts = histogram(layout, a)
        _, _, n_esc = dictionary(layout, counts, a.size)
    cap = container_size(layout, a.size, n_esc, flags)
    out = np.zeros(cap, dtype=np.uint8)
    size = ctypes.c_uint64(0)
    if flags:
        st = _load().orc_encode_flags(layout, flags, _ptr(a), a.size, _ptr(out), cap,
                                      ctypes.byref(size))
    else:
        st = _load().orc_encode(layout, _ptr(a), a.size, _ptr(out), cap, ctypes.byref(size))
    _check(st, "encode")
    assert size.value == cap
    return out


def header_info(container: np.ndarray) -> dict:
    c = np.ascontiguousarray(container, dtype=np.uint8)
    lay = ctypes.c_int(0)
    nd = ctypes.c_int(0)
    n = ctypes.c_uint64(0)
    ne = ctypes.c_uint64(0)
    d = np.zeros(16, dtype=np.uint16)
    off = np.zeros(6, dtype=np.uint64)
    _check(_load().orc_header_info(_ptr(c), c.size, ctypes.byref(lay), ctypes.byref(nd),
                                   ctypes.byref(n), ctypes.byref(ne), _ptr(d), _ptr(off)),
           "header")
    fl = ctypes.c_int(0)
    _check(_load().orc_header_flags(_ptr(c), c.size, ctypes.byref(fl)), "header")
    return {"layout": lay.value, "flags": fl.value, "n_dict": nd.value, "n": n.value,
            "n_esc": ne.value,
            "dict": d, "off_codes": int(off[0]), "off_raw": int(off[1]),
            "off_esc_pos": int(off[2]), "off_esc_sym": int(off[3]),
            "total_bytes": int(off[4]), "off_esc_idx": int(off[5])}


def decode(container: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(container, dtype=np.uint8)
    n = header_info(c)["n"]
    out = np.zeros(n, dtype=np.uint16)
    _check(_load().orc_decode(_ptr(c), c.size, _ptr(out), n), "decode")
    return out


def _gemv_args(W, x):
    W = np.ascontiguousarray(W)
    x = np.ascontiguousarray(x)
    if W.dtype != np.uint16 or x.dtype != np.uint16 or W.ndim != 2:
        raise TypeError("W [rows, cols] and x [batch, cols] must be uint16 BF16 bit patterns")
    if x.ndim == 1:
        x = x.reshape(1, -1)
    if x.shape[1] != W.shape[1]:
        raise ValueError("x columns must match W columns")
    return W, x


def gemv_f32(W, x) -> np.ndarray:
    """y[b, r] = sum_c f32(W[r, c]) * f32(x[b, c]), fp32, ascending c."""
    W, x = _gemv_args(W, x)
    y = np.zeros((x.shape[0], W.shape[0]), dtype=np.float32)
    _check(_load().orc_gemv_f32(_ptr(W), W.shape[0], W.shape[1], _ptr(x), x.shape[0],
                                _ptr(y)), "gemv_f32")
    return y


def gemv_f64(W, x):
    """(y, a): the same sum in fp64 and a = sum_c |W[r, c] x[b, c]|."""
    W, x = _gemv_args(W, x)
    y = np.zeros((x.shape[0], W.shape[0]), dtype=np.float64)
    a = np.zeros_like(y)
    _check(_load().orc_gemv_f64(_ptr(W), W.shape[0], W.shape[1], _ptr(x), x.shape[0],
                                _ptr(y), _ptr(a)), "gemv_f64")
    return y, a


def bits_per_weight(container: np.ndarray):
    c = np.ascontiguousarray(container, dtype=np.uint8)
    b = ctypes.c_double(0)
    p = ctypes.c_double(0)
    _check(_load().orc_bits_per_weight(_ptr(c), c.size, ctypes.byref(b), ctypes.byref(p)),
           "bits_per_weight")
    return b.value, p.value


def saving(bpw: float) -> float:
    """Size saving against BF16 for a bits/weight figure: 1 - bpw / 16."""
    return 1.0 - bpw / 16.0
