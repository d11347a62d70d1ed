"""The serialized artifact and its checksums, on the host (no GPU): CRC-32
against zlib's, per-region container CRCs, write/read round trips of oracle
containers, and a corruption suite in which every damaged region of the file
is reported as corrupt.  The pages ask for a serialized artifact with metadata
and escapes, for every tensor to be decoded from it and compared, and for
corruption to have a defined outcome (page "Compresión de pesos LLM sin
pérdida vs 8-bit GGUF: ¿qué está listo para producción?", sections "¿Está
listo para producción el resultado de GLM-5.2?" and "Preguntas para un vendor
o equipo de investigación")."""
import os
import zlib

import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module")
def wc():
    import decode_gemv_sign_amd
    return decode_gemv_sign_amd


def test_crc32_is_zlibs(wc):
    rng = np.random.default_rng(3)
    for n in (0, 1, 7, 8, 9, 15, 16, 17, 1000, 65537, 1 << 20):
        b = rng.integers(0, 256, n, dtype=np.uint8)
        assert wc.crc32(b) == zlib.crc32(b.tobytes()), n
    # the standard check value, and a continued computation
    assert wc.crc32(b"123456789") == 0xCBF43926
    b = rng.integers(0, 256, 5000, dtype=np.uint8)
    assert wc.crc32(b[3000:], wc.crc32(b[:3000])) == zlib.crc32(b.tobytes())


def _containers():
    """(name, shape, source, container) for a spread of oracle containers."""
    out = []
    d = synth.small()
    out.append(("small.bytesplit", d["W"].shape, d["W"], oracle.encode(oracle.BYTESPLIT, d["W"])))
    out.append(("small.k15", d["W"].shape, d["W"], oracle.encode(oracle.K15, d["W"])))
    out.append(("small.k15.compact", d["W"].shape, d["W"],
                oracle.encode(oracle.K15, d["W"], oracle.COMPACT)))
    u = synth.random_bits(3 * 4097, 11, "uniform").reshape(3, 4097)
    out.append(("uniform.raw", u.shape, u, oracle.encode(oracle.RAW, u)))
    e = np.full((2, 2, 2, 5), 0x3F80, dtype=np.uint16)  # no escapes, 4-d
    out.append(("const.4d", e.shape, e, oracle.encode(oracle.K15, e)))
    z = np.zeros(0, dtype=np.uint16)
    out.append(("empty", (0,), z, oracle.encode(oracle.BYTESPLIT, z)))
    return out


def test_container_crcs_cover_every_region(wc):
    for name, _, _, c in _containers():
        info = oracle.header_info(c)
        bounds = [0, 128, info["off_raw"], info["off_esc_pos"], info["off_esc_sym"],
                  info["off_esc_idx"], info["total_bytes"]]
        want = [zlib.crc32(c[bounds[k]:bounds[k + 1]].tobytes()) for k in range(6)]
        assert wc.container_crcs(c) == want, name


def _write(wc, path, items):
    wc.artifact_write(str(path), [(n, s, c, zlib.crc32(np.ascontiguousarray(src).tobytes()))
                                  for n, s, src, c in items])


def test_artifact_round_trip(wc, tmp_path):
    items = _containers()
    path = tmp_path / "a.wca"
    _write(wc, path, items)
    ents = wc.artifact_entries(str(path))
    assert [e["name"] for e in ents] == [it[0] for it in items]
    for e, (name, shape, src, c) in zip(ents, items):
        assert e["shape"] == tuple(shape)
        assert e["offset"] % 4096 == 0 and e["bytes"] == c.size
        assert e["layout"] == oracle.header_info(c)["layout"]
        assert e["src_crc"] == zlib.crc32(np.ascontiguousarray(src).tobytes())
    for i, (_, _, src, c) in enumerate(items):
        got = wc.artifact_read(str(path), i)
        assert np.array_equal(got, c)
        assert np.array_equal(oracle.decode(got), np.ascontiguousarray(src).reshape(-1))
    # the file: header, table, then containers at 4096-byte offsets with zero gaps
    raw = np.fromfile(path, dtype=np.uint8)
    assert raw[:4].tobytes() == b"WCA1"
    assert raw.size == ents[-1]["offset"] + ents[-1]["bytes"]
    # an empty artifact
    wc.artifact_write(str(tmp_path / "e.wca"), [])
    assert wc.artifact_entries(str(tmp_path / "e.wca")) == []


def _code(wc, fn):
    with pytest.raises(wc.WCError) as e:
        fn()
    return e.value.code


def test_corruption_is_detected(wc, tmp_path):
    items = _containers()
    path = tmp_path / "a.wca"
    _write(wc, path, items)
    good = np.fromfile(path, dtype=np.uint8)
    ents = wc.artifact_entries(str(path))
    # one flipped bit in each place: the file header, each entry, and every
    # region of every container
    spots = [("file header", 9), ("header crc", 61)]
    for i in range(len(items)):
        base = 64 + 256 * i
        spots += [(f"entry {i} name", base + 1), (f"entry {i} shape", base + 104),
                  (f"entry {i} offset", base + 137), (f"entry {i} crc", base + 253)]
    # the zero gaps: after the table, and after each container but the last
    spots.append(("gap after the table", 64 + 256 * len(items)))
    for e in ents[:-1]:
        if (e["offset"] + e["bytes"]) % 4096:
            spots.append((f"gap after {e['name']}", e["offset"] + e["bytes"]))
    for i, e in enumerate(ents):
        c = items[i][3]
        info = oracle.header_info(c)
        bounds = [0, 128, info["off_raw"], info["off_esc_pos"], info["off_esc_sym"],
                  info["off_esc_idx"], info["total_bytes"]]
        for k in range(6):
            if bounds[k + 1] > bounds[k]:
                spots.append((f"{e['name']} region {k}", e["offset"] + (bounds[k] + bounds[k + 1]) // 2))
    for what, off in spots:
        bad = good.copy()
        bad[off] ^= 0x10
        p = tmp_path / "bad.wca"
        bad.tofile(p)
        codes = set()
        try:
            ents_b = wc.artifact_entries(str(p))
            for i in range(len(ents_b)):
                try:
                    wc.artifact_read(str(p), i)
                except wc.WCError as err:
                    codes.add(err.code)
        except wc.WCError as err:
            codes.add(err.code)
        assert codes == {-3}, (what, codes)
    # truncated, and with a byte appended
    for bad in (good[:-1], np.concatenate([good, np.zeros(1, np.uint8)])):
        p = tmp_path / "bad.wca"
        bad.tofile(p)
        assert _code(wc, lambda: wc.artifact_entries(str(p))) == -3
    # a missing file
    assert _code(wc, lambda: wc.artifact_entries(str(tmp_path / "none.wca"))) == -6


def test_writer_rejects_bad_input(wc, tmp_path):
    name, shape, src, c = _containers()[0]
    p = str(tmp_path / "w.wca")
    crc = zlib.crc32(src.tobytes())
    assert _code(wc, lambda: wc.artifact_write(p, [("x" * 96, shape, c, crc)])) == -1
    assert _code(wc, lambda: wc.artifact_write(p, [(name, (3, 5), c, crc)])) == -1
    bad = c.copy()
    bad[6] = 7  # layout byte
    assert _code(wc, lambda: wc.artifact_write(p, [(name, shape, bad, crc)])) == -3
    assert not os.path.exists(p)
