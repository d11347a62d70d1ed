"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * hand-derived golden containers and a hand-worked GEMV (tests/golden/);
  * the lossless criterion the pages use — every tensor rebuilt bit for bit —
    on all 65,536 BF16 bit patterns and on random tensors of ragged sizes
    (page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%", section
    "Cómo funciona la compresión");
  * brute force on small inputs: collections.Counter histograms and a
    sorted()-based top-15 (a different algorithm from the oracle's repeated
    selection);
  * the pages' accounting decomposition (4 code bits + 8 raw bits for
    byte-split, 4 + 7 for K15, plus escape overhead) and the pages' printed
    totals (12.005 b/w <-> 24.967%, 11.173 b/w <-> 30.168%, 1,403.19 GiB ->
    979.87 GiB), same page and section;
  * exact GEMV cases (one-hot inputs, small integers) and float64 matmul;
  * planted mistakes: copies of the oracle with one plausible bug each must
    fail at least one of these pins.
"""
import collections
import json
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth
from tests.tolerance import assert_gemv_close

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "containers.json")))["cases"]
GEMV_GOLDEN = json.load(open(os.path.join(HERE, "golden", "gemv.json")))
LAYOUTS = [oracle.BYTESPLIT, oracle.K15]


def _hex(s):
    return bytes.fromhex(re.sub(r"\s+", "", s))


def expected_container(case):
    buf = bytearray(case["total_bytes"])
    for off, hx in case["header"].items():
        b = _hex(hx)
        buf[int(off):int(off) + len(b)] = b
    for off, hx in case["streams"].items():
        b = _hex(hx)
        buf[int(off):int(off) + len(b)] = b
    return bytes(buf)


def weights_of(case):
    if "weights_sparse" in case:
        sp = case["weights_sparse"]
        w = np.full(sp["n"], int(sp["fill"], 16), dtype=np.uint16)
        for i, h in sp["at"].items():
            w[int(i)] = int(h, 16)
        return w
    return np.array([int(h, 16) for h in case["weights"]], dtype=np.uint16)


def shift_of(layout):
    return 7 if layout == oracle.K15 else 8


# ---------------------------------------------------------------- golden

@pytest.mark.parametrize("case", GOLDEN, ids=[c["name"] for c in GOLDEN])
def test_golden_container_bytes(case):
    w = weights_of(case)
    got = oracle.encode(case["layout"], w).tobytes()
    exp = expected_container(case)
    assert len(got) == case["total_bytes"]
    assert got == exp, (got.hex(), exp.hex())


@pytest.mark.parametrize("case", GOLDEN, ids=[c["name"] for c in GOLDEN])
def test_golden_header_and_decode(case):
    c = np.frombuffer(expected_container(case), dtype=np.uint8)
    info = oracle.header_info(c)
    assert info["n_dict"] == case["n_dict"]
    assert info["n_esc"] == case["n_esc"]
    exp_dict = [int(h, 16) for h in case["dict"]] + [0] * (16 - len(case["dict"]))
    assert list(info["dict"]) == exp_dict
    assert np.array_equal(oracle.decode(c), weights_of(case))
    if case["bpw"] is not None:
        bpw, pay = oracle.bits_per_weight(c)
        assert bpw == pytest.approx(case["bpw"], rel=1e-12)
        assert pay == pytest.approx(case["payload_bpw"], rel=1e-12)


def test_golden_gemv():
    W = np.array([[int(h, 16) for h in r] for r in GEMV_GOLDEN["W"]], dtype=np.uint16)
    x = np.array([[int(h, 16) for h in r] for r in GEMV_GOLDEN["x"]], dtype=np.uint16)
    y = np.array(GEMV_GOLDEN["y"], dtype=np.float32)
    assert np.array_equal(oracle.gemv_f32(W, x), y)
    y64, _ = oracle.gemv_f64(W, x)
    assert np.array_equal(y64, y.astype(np.float64))


# ------------------------------------------------- lossless round trips

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("shuffle", [None, 7])
def test_roundtrip_all_bit_patterns(layout, shuffle):
    w = synth.all_patterns(shuffle)
    c = oracle.encode(layout, w)
    assert np.array_equal(oracle.decode(c), w)
    info = oracle.header_info(c)
    nsym = 512 if layout == oracle.K15 else 256
    # every symbol occurs equally often; the 15 smallest symbols are kept
    assert info["n_dict"] == 15
    assert list(info["dict"][:15]) == list(range(15))
    assert info["n_esc"] == (nsym - 15) * (65536 // nsym)


SIZES = [0, 1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1000, 2047,
         2048, 2049, 8191, 8193, 20001]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("kind", ["normal", "uniform", "few"])
def test_roundtrip_ragged_sizes(layout, kind):
    for i, n in enumerate(SIZES):
        w = synth.random_bits(n, seed=100 + i, kind=kind)
        c = oracle.encode(layout, w)
        assert c.size == oracle.container_size(layout, n, oracle.header_info(c)["n_esc"])
        assert np.array_equal(oracle.decode(c), w), (layout, kind, n)


# ------------------------------------------- brute-force counts and ranks

@pytest.mark.parametrize("layout", LAYOUTS)
def test_histogram_brute_force(layout):
    for seed, kind, n in [(1, "normal", 3000), (2, "uniform", 5000), (3, "few", 999)]:
        w = synth.random_bits(n, seed, kind)
        got = oracle.histogram(layout, w)
        cnt = collections.Counter(int(b) >> shift_of(layout) for b in w)
        exp = np.zeros(len(got), dtype=np.uint64)
        for s, k in cnt.items():
            exp[s] = k
        assert np.array_equal(got, exp)
        assert int(got.sum()) == n


def test_bytesplit_histogram_is_pair_sum_of_k15():
    w = synth.random_bits(50000, 5, "uniform")
    h9 = oracle.histogram(oracle.K15, w)
    h8 = oracle.histogram(oracle.BYTESPLIT, w)
    assert np.array_equal(h8, h9[0::2] + h9[1::2])


def _brute_dict(w, layout):
    cnt = collections.Counter(int(b) >> shift_of(layout) for b in w)
    ranked = sorted(cnt.items(), key=lambda kv: (-kv[1], kv[0]))[:15]
    return [s for s, _ in ranked], len(w) - sum(k for _, k in ranked)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_dictionary_brute_force(layout):
    for seed, kind, n in [(11, "normal", 4000), (12, "uniform", 4000), (13, "few", 300),
                          (14, "normal", 1), (15, "uniform", 17)]:
        w = synth.random_bits(n, seed, kind)
        d, nd, ne = oracle.dictionary(layout, oracle.histogram(layout, w), n)
        exp, exp_ne = _brute_dict(w, layout)
        assert list(d[:nd]) == exp and nd == len(exp) and ne == exp_ne
        assert all(v == 0 for v in d[nd:])


def test_dictionary_hand_cases():
    bs = oracle.BYTESPLIT
    # (i) at most 15 distinct symbols: nothing escapes
    w = np.array([(s << 8) | 1 for s in range(15) for _ in range(s + 1)], dtype=np.uint16)
    d, nd, ne = oracle.dictionary(bs, oracle.histogram(bs, w), w.size)
    assert nd == 15 and ne == 0
    # (ii) 16 symbols with distinct counts: exactly the rarest escapes
    w = np.array([(s << 8) for s in range(16) for _ in range(20 - s)], dtype=np.uint16)
    d, nd, ne = oracle.dictionary(bs, oracle.histogram(bs, w), w.size)
    assert list(d[:15]) == list(range(15)) and ne == 20 - 15
    # (iii) 16 equal counts: the largest symbol escapes
    w = np.array([(s << 8) for s in range(0x40, 0x50) for _ in range(3)], dtype=np.uint16)
    d, nd, ne = oracle.dictionary(bs, oracle.histogram(bs, w), w.size)
    assert list(d[:15]) == list(range(0x40, 0x4F)) and ne == 3
    # (iv) constant tensor
    w = np.full(77, 0xBEEF, dtype=np.uint16)
    d, nd, ne = oracle.dictionary(bs, oracle.histogram(bs, w), w.size)
    assert nd == 1 and d[0] == 0xBE and ne == 0


@pytest.mark.parametrize("layout", LAYOUTS)
def test_top15_property(layout):
    w = synth.random_bits(100000, 21, "uniform")
    h = oracle.histogram(layout, w)
    d, nd, ne = oracle.dictionary(layout, h, w.size)
    last = int(h[d[nd - 1]])
    inside = set(int(s) for s in d[:nd])
    for s in range(len(h)):
        if s not in inside and h[s]:
            assert h[s] < last or (h[s] == last and s > d[nd - 1])


# ---------------------------------------------------- escape stream (P6)

def _streams(c):
    info = oracle.header_info(c)
    lay = info["layout"]
    e = info["n_esc"]
    codes = c[info["off_codes"]:info["off_codes"] + (info["n"] + 1) // 2]
    pos = c[info["off_esc_pos"]:info["off_esc_pos"] + 4 * e].view("<u4")
    sb = 2 if lay == oracle.K15 else 1
    sym = c[info["off_esc_sym"]:info["off_esc_sym"] + sb * e].view("<u2" if sb == 2 else "u1")
    return info, codes, pos, sym


@pytest.mark.parametrize("layout", LAYOUTS)
def test_escape_stream_invariants(layout):
    d = synth.banded(rows=256, cols=512, bands=1, band_rows=64, batch=1)
    for w in (d["W"].reshape(-1), synth.random_bits(30000, 31, "uniform"),
              synth.random_bits(30000, 32, "normal", sigma=3.0)):
        c = oracle.encode(layout, w)
        info, codes, pos, sym = _streams(c)
        sh = shift_of(layout)
        # one nibble equal to 15 per escape (count is independent of nibble order)
        n15 = int(np.sum((codes & 15) == 15) + np.sum((codes >> 4) == 15))
        assert n15 == info["n_esc"]
        assert np.all(np.diff(pos.astype(np.int64)) > 0)
        assert np.array_equal(sym.astype(np.uint32), w[pos].astype(np.uint32) >> sh)
        dset = set(int(s) for s in info["dict"][:info["n_dict"]])
        assert not any(int(s) in dset for s in sym)
        exp_pos = np.nonzero(~np.isin(w.astype(np.uint32) >> sh, list(dset)))[0]
        assert np.array_equal(pos.astype(np.int64), exp_pos)
        # index entry j = escapes below weight 2048 j, for every tile start and
        # the last tile's end (counted here by a search of the positions)
        tiles = -(-w.size // 2048)
        idx = c[info["off_esc_idx"]:info["off_esc_idx"] + 4 * (tiles + 1)].view("<u4")
        bounds = 2048 * np.arange(tiles + 1, dtype=np.int64)
        assert np.array_equal(idx.astype(np.int64), np.searchsorted(exp_pos, bounds, "left"))
        assert info["total_bytes"] == -(-(info["off_esc_idx"] + 4 * (tiles + 1)) // 16) * 16


# ------------------------------------------------ raw layout and choice

def test_raw_roundtrip_and_accounting():
    for i, n in enumerate([0, 1, 7, 8, 9, 2047, 2048, 20001]):
        w = synth.random_bits(n, 900 + i, "uniform")
        c = oracle.encode(oracle.RAW, w)
        info = oracle.header_info(c)
        assert (info["layout"], info["n_dict"], info["n_esc"]) == (oracle.RAW, 0, 0)
        assert c.size == 128 + -(-2 * n // 16) * 16
        assert np.array_equal(c[128:128 + 2 * n].view("<u2"), w)
        assert np.array_equal(oracle.decode(c), w)
        if n:
            bpw, pay = oracle.bits_per_weight(c)
            assert pay == 16.0 and bpw == 8 * c.size / n
    w = synth.all_patterns(5)
    assert np.array_equal(oracle.decode(oracle.encode(oracle.RAW, w)), w)


def _choice_cases():
    """(name, weights, expected layout) worked out by hand from the container
    sizes: header 128, codes ceil(n/2), raw n / ceil(7n/8) / 2n, 4 + 1 or 2
    bytes per escape, index 4 (tiles + 1) bytes with escapes, each padded to 16."""
    # one symbol: byte-split 128 + 2048 + 4096 = 6272, K15 128 + 2048 + 3584 =
    # 5760, raw 128 + 8192 = 8320
    const = np.full(4096, 0x3F80, dtype=np.uint16)
    # 30 exponents (100 weights each), 15 high bytes: byte-split has no
    # escapes (128 + 1504 + 3008 = 4640); K15 escapes 1500 of 3000 weights
    # (over 12000 bytes); raw 128 + 6000 = 6128
    e = np.repeat(np.arange(100, 130, dtype=np.uint16), 100)
    thirty = (e << 7) | np.uint16(0x15)
    # uniform bit patterns: nearly every weight escapes in both coded layouts
    uni = synth.random_bits(4096, 77, "uniform")
    # empty: every container is the 128-byte header; the tie goes to byte-split
    empty = np.zeros(0, dtype=np.uint16)
    return [("constant", const, oracle.K15), ("thirty_exponents", thirty, oracle.BYTESPLIT),
            ("uniform", uni, oracle.RAW), ("empty", empty, oracle.BYTESPLIT)]


@pytest.mark.parametrize("case", _choice_cases(), ids=lambda c: c[0] if isinstance(c, tuple) else "")
def test_layout_choice_hand_cases(case):
    _, w, want = case
    assert oracle.choose_layout(w) == want


def test_layout_choice_is_the_smallest_container():
    tensors = [synth.random_bits(n, 950 + n, kind) for n in (1, 100, 5000, 40000)
               for kind in ("normal", "uniform", "few")]
    tensors.append(synth.random_bits(6000, 3, "normal", sigma=300.0))  # wide exponent spread
    for w in tensors:
        sizes = [oracle.encode(lay, w).size for lay in (oracle.BYTESPLIT, oracle.K15, oracle.RAW)]
        assert oracle.choose_layout(w) == int(np.argmin(sizes)), sizes  # argmin: first of equals


# ------------------------------------------------------------- accounting

@pytest.mark.parametrize("layout", LAYOUTS)
def test_accounting_decomposition(layout):
    """Payload bits/weight = 4 (code) + 8 or 7 (raw) + escape bits (a 32-bit
    position and the symbol per escape, plus one 32-bit index entry per
    2048-weight tile and one closing entry when there are escapes); all
    overhead (header, padding) on top of that."""
    raw_bits = 7 if layout == oracle.K15 else 8
    esc_bits = 32 + (16 if layout == oracle.K15 else 8)
    for n, kind in [(4096, "normal"), (8192, "uniform"), (65536, "few"), (2 ** 20, "normal")]:
        w = synth.random_bits(n, n, kind)
        c = oracle.encode(layout, w)
        e = oracle.header_info(c)["n_esc"]
        bpw, pay = oracle.bits_per_weight(c)
        index_bits = 32 * (-(-n // 2048) + 1) if e else 0
        assert pay == pytest.approx(4 + raw_bits + (esc_bits * e + index_bits) / n, rel=1e-12)
        overhead_bytes = (bpw - pay) * n / 8
        assert 128 <= overhead_bytes < 128 + 5 * 16


def test_pages_printed_totals():
    # byte-split, validated: 12.005 bits/weight <-> 24.967% saving
    assert oracle.saving(12.005) == pytest.approx(0.24967, abs=5e-5)
    # K15 accounting: 11.173 bits/weight <-> 30.168% saving
    assert oracle.saving(11.173) == pytest.approx(0.30168, abs=5e-5)
    # 1,403.19 GiB -> 979.87 GiB is the same 30.168% saving
    assert 1 - 979.87 / 1403.19 == pytest.approx(0.30168, abs=5e-5)
    # ... and 1,403.19 GiB of BF16 is about 753e9 weights
    assert 1403.19 * 2 ** 30 / 2 == pytest.approx(753e9, rel=2e-3)


# -------------------------------------------------------------- GEMV pins

def test_gemv_one_hot_columns():
    rng = np.random.default_rng(3)
    W = synth.random_bits(64 * 48, 9, "normal").reshape(64, 48)
    for j in (0, 1, 17, 47):
        x = np.zeros((1, 48), dtype=np.uint16)
        x[0, j] = 0x3F80  # 1.0
        y = oracle.gemv_f32(W, x)
        assert np.array_equal(y[0].view(np.uint32), synth.bf16_to_f32(W[:, j]).view(np.uint32))
    # a square matrix, so a transposed product would still be shape-correct
    S = synth.random_bits(40 * 40, 10, "normal").reshape(40, 40)
    x = np.zeros((1, 40), dtype=np.uint16)
    x[0, 5] = 0x4000  # 2.0
    assert np.array_equal(oracle.gemv_f32(S, x)[0], 2 * synth.bf16_to_f32(S[:, 5]))
    del rng


def test_gemv_small_integers_exact():
    rng = np.random.default_rng(4)
    Wi = rng.integers(-8, 9, size=(37, 129))
    xi = rng.integers(-8, 9, size=(3, 129))
    W = synth.bf16_bits(Wi.astype(np.float32)).reshape(Wi.shape)
    x = synth.bf16_bits(xi.astype(np.float32)).reshape(xi.shape)
    exp = (xi @ Wi.T).astype(np.float64)
    assert np.array_equal(oracle.gemv_f32(W, x).astype(np.float64), exp)
    assert np.array_equal(oracle.gemv_f64(W, x)[0], exp)


def test_gemv_against_float64_matmul():
    d = synth.small()
    W, x = d["W"][:256], d["x"]
    Wf = synth.bf16_to_f32(W).astype(np.float64)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    ref = xf @ Wf.T
    a = np.abs(xf) @ np.abs(Wf).T
    y64, a64 = oracle.gemv_f64(W, x)
    assert np.all(np.abs(y64 - ref) <= 1e-12 * a)
    assert np.allclose(a64, a, rtol=1e-12)
    assert_gemv_close(oracle.gemv_f32(W, x), ref, a, "oracle fp32 vs float64 matmul")


def test_gemv_of_decoded_equals_gemv_of_original():
    d = synth.small()
    W = d["W"][:128]
    for layout in LAYOUTS:
        Wd = oracle.decode(oracle.encode(layout, W)).reshape(W.shape)
        assert np.array_equal(oracle.gemv_f32(Wd, d["x"]), oracle.gemv_f32(W, d["x"]))


# ------------------------------------------------------ corrupt containers

def _err(fn, *a):
    with pytest.raises(oracle.OracleError) as e:
        fn(*a)
    return e.value.code


@pytest.mark.parametrize("layout", LAYOUTS)
def test_corruption_detected(layout):
    w = synth.random_bits(3000, 41, "uniform")
    c = oracle.encode(layout, w)
    assert oracle.header_info(c)["n_esc"] > 0
    for off, val in [(0, 0x00), (4, 0x02), (6, 0x05), (7, 16), (56, 0x90), (64, 0x00),
                     (88, 0x00), (100, 0x01), (16, 0xFF)]:
        bad = c.copy()
        bad[off] = val if bad[off] != val else (val ^ 1)
        assert _err(oracle.decode, bad) == -3, off
    # truncated container
    assert _err(oracle.decode, c[:-16]) == -3
    # escape position moved: the record no longer sits at its weight
    info = oracle.header_info(c)
    for k in (1, 0):  # an index entry off by one (a tile start, then the first)
        bad = c.copy()
        bad[info["off_esc_idx"] + 4 * k] ^= 1
        assert _err(oracle.decode, bad) == -3, k
    bad = c.copy()
    bad[info["off_esc_pos"]] ^= 1
    assert _err(oracle.decode, bad) == -3
    # a dictionary code replaced by 15 without a record
    bad = c.copy()
    codes = bad[info["off_codes"]:]
    j = int(np.argmax((codes[:info["n"] // 2] & 15) != 15))
    codes[j] |= 15
    assert _err(oracle.decode, bad) == -3


# ------------------------------------------------------ generators (P9)

def test_generators_realized_structure():
    d = synth.small()
    assert d["scaled_positions"].size == 524
    d2 = synth.square()
    n = 4096 * 4096
    assert d2["zero_positions"].size == round(0.01 * n)
    assert d2["outlier_positions"].size == round(0.001 * n)
    assert np.all(d2["W"].reshape(-1)[d2["zero_positions"]] == 0)
    assert np.intersect1d(d2["zero_positions"], d2["outlier_positions"]).size == 0
    a = synth.small()["W"]
    assert np.array_equal(a, synth.small()["W"])  # seeded


def test_banded_escape_fraction():
    """The banded workload's byte-split escapes come out near 5% and sit almost
    all inside the 5 filled bands."""
    d = synth.banded()
    w = d["W"].reshape(-1)
    h = oracle.histogram(oracle.BYTESPLIT, w)
    dct, nd, ne = oracle.dictionary(oracle.BYTESPLIT, h, w.size)
    frac = ne / w.size
    assert 0.048 <= frac <= 0.052, frac
    dset = np.isin(w >> 8, dct[:nd])
    rows_esc = (~dset).reshape(d["W"].shape).sum(axis=1)
    in_band = sum(rows_esc[b * 64:(b + 1) * 64].sum() for b in d["bands"])
    assert in_band / ne > 0.98


# ------------------------------------------- planted mistakes are caught

# ---------------------------------------------- compact escape form (flags)
#
# The compact form drops the escape-position stream: the k-th weight whose
# code is 15 takes the k-th escape symbol.  Its expected container follows
# from a full one by the format's own definition (16-byte aligned streams,
# header fields at fixed offsets), written out here without the oracle.


def _le(b, off, size):
    return int.from_bytes(b[off:off + size], "little")


def compact_from_full(full: bytes) -> bytes:
    """The compact container with the same content as `full`: the position
    stream removed, the later streams moved up, the flag byte set."""
    pad = lambda x: (x + 15) // 16 * 16  # noqa: E731
    layout, n, n_esc = full[6], _le(full, 8, 8), _le(full, 16, 8)
    off_pos, off_sym, off_idx = _le(full, 72, 8), _le(full, 80, 8), _le(full, 96, 8)
    sym_len = n_esc * (2 if layout == oracle.K15 else 1)
    idx_len = 4 * ((n + 2047) // 2048 + 1) if n_esc else 0
    new_sym = off_pos
    new_idx = pad(new_sym + sym_len)
    total = pad(new_idx + idx_len)
    out = bytearray(total)
    out[:off_pos] = full[:off_pos]                  # header, codes, raw part
    out[new_sym:new_sym + sym_len] = full[off_sym:off_sym + sym_len]
    out[new_idx:new_idx + idx_len] = full[off_idx:off_idx + idx_len]
    out[80:88] = new_sym.to_bytes(8, "little")
    out[88:96] = total.to_bytes(8, "little")
    out[96:104] = new_idx.to_bytes(8, "little")
    out[104] = oracle.COMPACT
    return bytes(out)


CODED_GOLDEN = [c for c in GOLDEN if c["layout"] != oracle.RAW]


@pytest.mark.parametrize("case", CODED_GOLDEN, ids=[c["name"] for c in CODED_GOLDEN])
def test_compact_golden(case):
    """Compact encode equals the hand-derived golden with its positions
    removed; decoding it rebuilds the weights."""
    want = compact_from_full(expected_container(case))
    got = oracle.encode(case["layout"], weights_of(case), oracle.COMPACT)
    assert got.tobytes() == want
    assert oracle.header_info(got)["flags"] == oracle.COMPACT
    assert np.array_equal(oracle.decode(got), weights_of(case))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compact_roundtrip_and_structure(layout):
    """Every bit pattern, and ragged random tensors across several index
    tiles: exact round trip, and the compact container is the full one
    without its positions."""
    cases = [synth.all_patterns(5)] + [synth.random_bits(n, 40 + n % 7, kind)
                                       for n, kind in ((1, "normal"), (2049, "uniform"),
                                                       (6150, "normal"), (10007, "uniform"))]
    for w in cases:
        full = oracle.encode(layout, w)
        comp = oracle.encode(layout, w, oracle.COMPACT)
        assert comp.tobytes() == compact_from_full(full.tobytes())
        assert np.array_equal(oracle.decode(comp), w)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compact_accounting(layout):
    """The compact payload is the full one less 32 bits per escape."""
    w = synth.random_bits(20000, 77, "uniform")
    full = oracle.encode(layout, w)
    comp = oracle.encode(layout, w, oracle.COMPACT)
    n_esc = oracle.header_info(full)["n_esc"]
    assert n_esc > 0
    _, pay_full = oracle.bits_per_weight(full)
    _, pay_comp = oracle.bits_per_weight(comp)
    assert pay_full - pay_comp == pytest.approx(32.0 * n_esc / w.size, rel=1e-12)
    assert oracle.container_size(layout, w.size, n_esc, oracle.COMPACT) == comp.size


def test_compact_rejects():
    w = synth.random_bits(3000, 78, "uniform")
    with pytest.raises(oracle.OracleError):
        oracle.encode(oracle.RAW, w, oracle.COMPACT)
    with pytest.raises(oracle.OracleError):
        oracle.encode(oracle.K15, w, 2)
    full = oracle.encode(oracle.K15, w)
    bad = full.copy()
    bad[104] = oracle.COMPACT  # the flag without moving the streams
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode(bad)
    assert e.value.code == -3
    comp = oracle.encode(oracle.K15, w, oracle.COMPACT)
    bad = comp.copy()
    bad[104] = 3
    with pytest.raises(oracle.OracleError):
        oracle.decode(bad)


MUTATIONS = {
    "nibble_order": [(r"\(i % 2\) \* 4", "(1 - i % 2) * 4")],
    "tie_break": [(r"counts\[s\] > counts\[best\]", "counts[s] >= counts[best]")],
    "k15_bit_order": [(r"7u \* i \+ \(uint64_t\)k", "7u * i + (uint64_t)(6 - k)")],
    "escape_symbol": [(r"put_le\(esc_sym \+ sym_bytes\(layout\) \* e, s,",
                       "put_le(esc_sym + sym_bytes(layout) * e, s ^ 1u,")],
    "padding": [(r"return \(x \+ 15u\) / 16u \* 16u;", "return (x + 7u) / 8u * 8u;")],
    "gemv_transposed": [(r"bf16_to_f32\(W\[r \* cols \+ c\]\) \* bf16_to_f32",
                         "bf16_to_f32(W[c * rows + r]) * bf16_to_f32")],
    "gemv_dropped_term": [(r"float acc = 0\.0f;\n      for \(uint64_t c = 0;",
                           "float acc = 0.0f;\n      for (uint64_t c = 1;")],
    "symbol_shift": [(r"return layout == ORC_LAYOUT_K15 \? 7 : 8;", "return layout == ORC_LAYOUT_K15 ? 8 : 8;")],
    # index entries counted up to and including the tile's first weight, in
    # the encoder and in the decoder's check alike
    "raw_byte_order": [(r"put_le\(out \+ off\[1\] \+ 2u \* i, w\[i\], 2\);",
                        "put_le(out + off[1] + 2u * i, (uint16_t)((w[i] >> 8) | (w[i] << 8)), 2);"),
                       (r"out\[i\] = \(uint16_t\)get_le\(c \+ off\[1\] \+ 2u \* i, 2\);",
                        "{ uint16_t v = (uint16_t)get_le(c + off[1] + 2u * i, 2); out[i] = (uint16_t)((v >> 8) | (v << 8)); }")],
    "choice_tie": [(r"if \(best < 0 \|\| total < best_total\)", "if (best < 0 || total <= best_total)")],
    "compact_keeps_positions": [(r"return \(flags & ORC_FLAG_COMPACT\) \? 0u : 4u \* e;", "return 4u * e;")],
    "index_inclusive": [(r"if \(n_esc && i % ORC_INDEX_TILE == 0\) put_le\(esc_idx \+ 4u \* \(i / ORC_INDEX_TILE\), e, 4\);\n    uint32_t s = symbol_of\(layout, w\[i\]\);",
                         "uint32_t s = symbol_of(layout, w[i]);\n    if (n_esc && i % ORC_INDEX_TILE == 0) put_le(esc_idx + 4u * (i / ORC_INDEX_TILE), e + (code_of[s] == 15), 4);"),
                        (r"get_le\(esc_idx \+ 4u \* \(i / ORC_INDEX_TILE\), 4\) != e\)",
                         "get_le(esc_idx + 4u * (i / ORC_INDEX_TILE), 4) != e + (((codes[i / 2] >> ((i % 2) * 4)) & 15u) == 15u))")],
}


def _pins_pass():
    """Run a compact subset of the pins; True when all hold."""
    try:
        for case in GOLDEN:
            if oracle.encode(case["layout"], weights_of(case)).tobytes() != expected_container(case):
                return False
            c = np.frombuffer(expected_container(case), dtype=np.uint8)
            if not np.array_equal(oracle.decode(c), weights_of(case)):
                return False
        W = np.array([[int(h, 16) for h in r] for r in GEMV_GOLDEN["W"]], dtype=np.uint16)
        x = np.array([[int(h, 16) for h in r] for r in GEMV_GOLDEN["x"]], dtype=np.uint16)
        if not np.array_equal(oracle.gemv_f32(W, x), np.array(GEMV_GOLDEN["y"], np.float32)):
            return False
        S = synth.random_bits(40 * 40, 10, "normal").reshape(40, 40)
        x = np.zeros((1, 40), dtype=np.uint16)
        x[0, 5] = 0x3F80
        if not np.array_equal(oracle.gemv_f32(S, x)[0], synth.bf16_to_f32(S[:, 5])):
            return False
        for layout in LAYOUTS:
            w = synth.all_patterns(3)
            if not np.array_equal(oracle.decode(oracle.encode(layout, w)), w):
                return False
        for _, w, want in _choice_cases():
            if oracle.choose_layout(w) != want:
                return False
        for case in CODED_GOLDEN:
            got = oracle.encode(case["layout"], weights_of(case), oracle.COMPACT)
            if got.tobytes() != compact_from_full(expected_container(case)):
                return False
    except oracle.OracleError:
        return False
    return True


def test_unmutated_oracle_passes_compact_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(HERE), "oracle", "wc_oracle.c")).read()
    mutated = src
    for pat, rep in MUTATIONS[name]:
        mutated, k = re.subn(pat, rep, mutated)
        assert k > 0, f"mutation {name} did not apply"
    shutil.copy(os.path.join(os.path.dirname(HERE), "oracle", "wc_oracle.h"), tmp_path)
    csrc = tmp_path / "wc_oracle.c"
    csrc.write_text(mutated)
    lib = str(tmp_path / "libmut.so")
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", str(csrc), "-o", lib])
    oracle.use_library(lib)
    try:
        assert not _pins_pass(), f"planted mistake '{name}' went unnoticed"
    finally:
        oracle.use_library(None)
