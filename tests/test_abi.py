"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and its host-only paths (header checks, accounting, argument checks
that fail before any device work) behave as include/wc.h states."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wc.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|double|uint32_t)\s+(wc_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def wc():
    import decode_gemv_sign_amd
    return decode_gemv_sign_amd


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "wc_build_dict", "wc_encode", "wc_encode_noalloc", "wc_decode", "wc_decode_gemv",
        "wc_gemv_bf16",
        "wc_bits_per_weight", "wc_crc32", "wc_container_crcs", "wc_artifact_write",
        "wc_artifact_count", "wc_artifact_entry", "wc_artifact_read"])


def test_library_exports_every_declared_symbol(wc):
    out = subprocess.check_output(["nm", "-D", "--defined-only", wc.LIB_PATH], text=True)
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(ctypes.CDLL(wc.LIB_PATH), name)


def test_library_is_gfx950_only(wc):
    # the offload bundle inside a hipcc shared library names its GPU targets
    blob = open(wc.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in blob


def _header_from_oracle(layout, w):
    import decode_gemv_sign_amd as wc
    c = oracle.encode(layout, w)
    return wc.Header.from_bytes(c[:128].tobytes()), c


@pytest.mark.parametrize("layout", [0, 1])
def test_bits_per_weight_matches_oracle(wc, layout):
    for n, kind in [(1, "normal"), (33, "uniform"), (5000, "normal"), (65536, "uniform")]:
        w = synth.random_bits(n, n, kind)
        h, c = _header_from_oracle(layout, w)
        assert wc.bits_per_weight(h) == pytest.approx(oracle.bits_per_weight(c), rel=1e-15)


def test_host_checks_reject_bad_headers(wc):
    w = synth.random_bits(3000, 5, "uniform")
    h, _ = _header_from_oracle(0, w)
    for field, val in [("magic", 0), ("version", 1), ("layout", 7), ("n_dict", 16),
                       ("off_raw", 0), ("total_bytes", 1), ("off_esc_idx", 0)]:
        bad = wc.Header.from_bytes(h.to_bytes())
        setattr(bad, field, val)
        with pytest.raises(wc.WCError) as e:
            wc.bits_per_weight(bad)
        assert e.value.code == -3, field
    bad = wc.Header.from_bytes(h.to_bytes())
    bad.reserved[3] = 1
    with pytest.raises(wc.WCError):
        wc.bits_per_weight(bad)
    bad = wc.Header.from_bytes(h.to_bytes())
    bad.dict[1] = bad.dict[0]  # duplicate dictionary entry
    with pytest.raises(wc.WCError):
        wc.bits_per_weight(bad)


def test_raw_layout_header(wc):
    w = synth.random_bits(1000, 6, "uniform")
    h, c = _header_from_oracle(2, w)
    assert (h.layout, h.n_dict, h.n_esc, h.off_raw, h.total_bytes) == (2, 0, 0, 128, 2128)
    bpw, pay = wc.bits_per_weight(h)
    assert pay == 16.0 and bpw == pytest.approx(8 * 2128 / 1000, rel=1e-15)
    for field, val in [("n_esc", 1), ("n_dict", 1), ("off_raw", 144)]:
        bad = wc.Header.from_bytes(h.to_bytes())
        setattr(bad, field, val)
        with pytest.raises(wc.WCError) as e:
            wc.bits_per_weight(bad)
        assert e.value.code == -3, field


def test_argument_checks_before_device_work(wc):
    lib = ctypes.CDLL(wc.LIB_PATH)
    lib.wc_build_dict.restype = ctypes.c_int
    h = wc.Header()
    # null workspace / null header / bad layout / n too large: no device call is made
    assert lib.wc_build_dict(0, None, ctypes.c_uint64(0), None, ctypes.c_size_t(0), None,
                             ctypes.byref(h)) == -1
    assert lib.wc_build_dict(0, None, ctypes.c_uint64(0), None, ctypes.c_size_t(0), None,
                             None) == -1
    assert lib.wc_build_dict(4, None, ctypes.c_uint64(0), None, ctypes.c_size_t(0), None,
                             ctypes.byref(h)) == -1
    assert lib.wc_build_dict(0, None, ctypes.c_uint64(1 << 32), None, ctypes.c_size_t(0), None,
                             ctypes.byref(h)) == -2
    # a zeroed header is corrupt for decode and GEMV
    assert lib.wc_decode(ctypes.byref(h), ctypes.c_void_p(16), ctypes.c_size_t(1 << 20),
                         ctypes.c_void_p(16), None) == -3
    # batch outside 1..256
    assert lib.wc_gemv_bf16(ctypes.c_void_p(16), ctypes.c_uint64(4), ctypes.c_uint64(32),
                            ctypes.c_void_p(16), ctypes.c_uint32(257), ctypes.c_void_p(16),
                            None) == -5
    assert lib.wc_gemv_bf16(ctypes.c_void_p(16), ctypes.c_uint64(4), ctypes.c_uint64(32),
                            ctypes.c_void_p(16), ctypes.c_uint32(0), ctypes.c_void_p(16),
                            None) == -5


def test_workspace_formula(wc, tmp_path):
    """The binding's workspace size equals the header's WC_WORKSPACE_BYTES(n),
    evaluated by a C program compiled against include/wc.h."""
    ns = (0, 1, 8191, 8192, 8193, 10 ** 9, (1 << 32) - 1)
    src = tmp_path / "ws.c"
    src.write_text('#include <stdio.h>\n#include "wc.h"\nint main(void){\n' +
                   "".join(f'printf("%zu\\n", WC_WORKSPACE_BYTES({n}ull));\n' for n in ns) +
                   "return 0;}\n")
    exe = tmp_path / "ws"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src),
                           "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)], text=True).split()]
    assert got == [wc.workspace_bytes(n) for n in ns]
    # counts and offsets (8 bytes) plus the symbol stage per 8192-weight block
    assert wc.workspace_bytes(8192) - wc.workspace_bytes(0) == 16 + 6 * wc.STAGE_SYMBOLS


def test_header_struct_layout(wc):
    offs = {f[0]: getattr(wc.Header, f[0]).offset for f in wc.Header._fields_}
    assert offs == {"magic": 0, "version": 4, "layout": 6, "n_dict": 7, "n": 8, "n_esc": 16,
                    "dict": 24, "off_codes": 56, "off_raw": 64, "off_esc_pos": 72,
                    "off_esc_sym": 80, "total_bytes": 88, "off_esc_idx": 96, "flags": 104,
                    "reserved": 105}
    # and a container header written by the oracle parses field by field
    w = np.array([0x3F80, 0xBF80, 0x3F80, 0x4000, 0x3F81], dtype=np.uint16)
    h, _ = _header_from_oracle(0, w)
    assert (h.magic, h.version, h.layout, h.n_dict, h.n, h.n_esc) == (0x36314357, 2, 0, 3, 5, 0)
    assert list(h.dict)[:3] == [0x3F, 0x40, 0xBF]
    assert (h.off_codes, h.off_raw, h.off_esc_pos, h.total_bytes, h.off_esc_idx) == \
        (128, 144, 160, 160, 160)


def test_compact_flag_in_header(wc):
    """Headers of the oracle's compact containers validate on the host, with
    the same accounting; an unknown flag, or the flag on the raw layout,
    does not."""
    w = synth.random_bits(30000, 9, "uniform")
    for layout in (0, 1):
        c = oracle.encode(layout, w, oracle.COMPACT)
        h = wc.Header.from_bytes(c[:128].tobytes())
        assert h.flags == wc.FLAG_COMPACT and h.off_esc_sym == h.off_esc_pos
        assert wc.bits_per_weight(h) == pytest.approx(oracle.bits_per_weight(c), rel=1e-15)
        bad = wc.Header.from_bytes(h.to_bytes())
        bad.flags = 2
        with pytest.raises(wc.WCError) as e:
            wc.bits_per_weight(bad)
        assert e.value.code == -3
        bad = wc.Header.from_bytes(h.to_bytes())
        bad.flags = 0  # the full form's offsets differ
        with pytest.raises(wc.WCError):
            wc.bits_per_weight(bad)
    h = wc.Header.from_bytes(oracle.encode(2, w)[:128].tobytes())
    h.flags = wc.FLAG_COMPACT
    with pytest.raises(wc.WCError):
        wc.bits_per_weight(h)
