"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars:
  * encode: every container byte identical to the oracle's;
  * decode: every weight bit-identical to the source (the pages' lossless
    criterion: page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%",
    section "Cómo funciona la compresión");
  * GEMV: per element |y - y_ref| <= 1e-3 max(|y_ref|, 2^-10 a) against the
    oracle's fp32 sequential sum and its fp64 sum (tests/tolerance.py), and
    bit-exact where the exact sum is representable (one-hot x, small integers).
Sizes: hand-derived golden containers, every BF16 bit pattern, ragged sizes
spanning several 2048-weight tiles, and the five workloads at full size in
the launch configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.test_oracle import GOLDEN, expected_container, weights_of
from tests.tolerance import assert_gemv_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_gemv_sign_amd as wc  # noqa: E402

DEV = "cuda:0"
LAYOUTS = [wc.BYTESPLIT, wc.K15]


def dev16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def host16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def gpu_encode(layout, w_np):
    w = dev16(w_np.reshape(-1))
    h, c = wc.encode(w, layout)
    torch.cuda.synchronize()
    return h, c


def check_roundtrip(layout, w_np, what):
    """GPU container == oracle container byte for byte; GPU decode exact."""
    w_flat = np.ascontiguousarray(w_np).reshape(-1)
    h, c = gpu_encode(layout, w_flat)
    ref = oracle.encode(layout, w_flat)
    got = c.cpu().numpy()
    assert got.size == ref.size, f"{what}: container size {got.size} vs {ref.size}"
    if not np.array_equal(got, ref):
        bad = np.nonzero(got != ref)[0]
        raise AssertionError(f"{what}: {bad.size} container bytes differ, first at {bad[0]} "
                             f"(gpu {got[bad[0]]:#x}, oracle {ref[bad[0]]:#x}); "
                             f"header says streams at codes={h.off_codes} raw={h.off_raw} "
                             f"pos={h.off_esc_pos} sym={h.off_esc_sym}")
    out = wc.decode(h, c)
    torch.cuda.synchronize()
    dec = host16(out)
    if not np.array_equal(dec, w_flat):
        bad = np.nonzero(dec != w_flat)[0]
        raise AssertionError(f"{what}: {bad.size} weights differ after decode, first at "
                             f"{bad[0]}: {dec[bad[0]]:#06x} vs {w_flat[bad[0]]:#06x}")
    return h, c


def oracle_gemv(W, x):
    y32 = oracle.gemv_f32(W, x)
    y64, a = oracle.gemv_f64(W, x)
    return y32, y64, a


def check_gemv(layout, W, x, h=None, c=None, what="", ref=None):
    """Fused decode-GEMV and the plain BF16 GEMV against the oracle.  `ref`
    may hold oracle results for a larger batch whose first rows are x."""
    rows, cols = W.shape
    batch = x.shape[0]
    if h is None:
        h, c = gpu_encode(layout, W)
    xd = dev16(x)
    y = wc.decode_gemv(h, c, rows, cols, xd)
    yb = wc.gemv_bf16(dev16(W), xd)
    torch.cuda.synchronize()
    y32, y64, a = oracle_gemv(W, x) if ref is None else (r[:batch] for r in ref)
    y = y.cpu().numpy()
    yb = yb.cpu().numpy()
    assert_gemv_close(y, y32, a, f"{what} fused vs oracle fp32")
    assert_gemv_close(y, y64, a, f"{what} fused vs oracle fp64")
    assert_gemv_close(yb, y64, a, f"{what} plain bf16 vs oracle fp64")
    return y, yb


# ------------------------------------------------------------ golden / exact

@pytest.mark.parametrize("case", GOLDEN, ids=[c["name"] for c in GOLDEN])
def test_golden_containers_on_gpu(case):
    w = weights_of(case)
    h, c = gpu_encode(case["layout"], w)
    assert c.cpu().numpy().tobytes() == expected_container(case)
    assert h.to_bytes() == expected_container(case)[:128]
    out = wc.decode(h, c)
    torch.cuda.synchronize()
    assert np.array_equal(host16(out), w)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("shuffle", [None, 7])
def test_all_bit_patterns(layout, shuffle):
    check_roundtrip(layout, synth.all_patterns(shuffle), f"all patterns shuffle={shuffle}")


RAGGED = [1, 2, 3, 31, 32, 33, 63, 64, 65, 2047, 2048, 2049, 6143, 8191, 8192, 8193, 20001,
          65537, 1 << 20, (1 << 20) + 7, 3 * 8192 * 64 + 1234]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("kind", ["normal", "uniform", "few"])
def test_ragged_sizes(layout, kind):
    for i, n in enumerate(RAGGED):
        check_roundtrip(layout, synth.random_bits(n, 500 + i, kind), f"{kind} n={n}")


# Tensors of 6146, 9301 and 12290 tiles (2048 weights each, the last one
# partial): the decode takes runs of 2 to 4 tiles per wave at the chip's wave
# counts, so its pipelined loops run every length with a ragged last run;
# 'normal' tensors take the three-slot ring and 'uniform' ones (almost every
# weight escapes) the two-slot ring.
LONG = [6145 * 2048 + 1001, 9300 * 2048 + 17, 12289 * 2048 + 2047]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("kind", ["normal", "uniform"])
def test_run_lengths(layout, kind):
    for i, n in enumerate(LONG):
        check_roundtrip(layout, synth.random_bits(n, 700 + i, kind), f"{kind} n={n}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_empty_tensor(layout):
    w = torch.empty(0, dtype=torch.int16, device=DEV)
    h, c = wc.encode(w, layout)
    torch.cuda.synchronize()
    assert h.n == 0 and h.total_bytes == 128
    assert np.array_equal(c.cpu().numpy(), oracle.encode(layout, np.zeros(0, np.uint16)))
    out = wc.decode(h, c)
    assert out.numel() == 0


def test_gemv_one_hot_exact():
    W = synth.random_bits(96 * 256, 3, "normal").reshape(96, 256)
    for layout in LAYOUTS:
        h, c = gpu_encode(layout, W)
        for j in (0, 31, 32, 255):
            x = np.zeros((1, 256), dtype=np.uint16)
            x[0, j] = 0x3F80
            y = wc.decode_gemv(h, c, 96, 256, dev16(x)).cpu().numpy()
            yb = wc.gemv_bf16(dev16(W), dev16(x)).cpu().numpy()
            exp = synth.bf16_to_f32(W[:, j])
            assert np.array_equal(y[0].view(np.uint32), exp.view(np.uint32)), (layout, j)
            assert np.array_equal(yb[0].view(np.uint32), exp.view(np.uint32)), (layout, j)


def test_gemv_small_integers_exact():
    rng = np.random.default_rng(4)
    for rows, cols, batch in [(37, 128, 3), (64, 2048, 16), (5, 4096 + 32, 4), (7, 100, 5)]:
        Wi = rng.integers(-8, 9, size=(rows, cols))
        xi = rng.integers(-8, 9, size=(batch, cols))
        W = synth.bf16_bits(Wi.astype(np.float32)).reshape(rows, cols)
        x = synth.bf16_bits(xi.astype(np.float32)).reshape(batch, cols)
        exp = (xi @ Wi.T).astype(np.float32)
        for layout in LAYOUTS:
            h, c = gpu_encode(layout, W)
            y = wc.decode_gemv(h, c, rows, cols, dev16(x)).cpu().numpy()
            assert np.array_equal(y, exp), (rows, cols, batch, layout)
        yb = wc.gemv_bf16(dev16(W), dev16(x)).cpu().numpy()
        assert np.array_equal(yb, exp)


# ------------------------------------------------ GEMV shapes and batches

@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemv_shapes_and_batches(layout):
    cases = [(1, 32, 1), (3, 64, 2), (65, 2048, 1), (17, 2080, 3), (33, 4096, 5), (9, 6144, 16),
             (40, 1000, 1), (11, 33, 7), (2, 1, 16), (128, 96, 4), (5, 24576, 8)]
    for i, (rows, cols, batch) in enumerate(cases):
        W = synth.random_bits(rows * cols, 700 + i, "normal").reshape(rows, cols)
        # sprinkle outliers so escapes land inside GEMV tiles
        W.reshape(-1)[::97] ^= 0x3000
        x = synth.vectors(800 + i, batch, cols)
        check_gemv(layout, W, x, what=f"{rows}x{cols} b={batch}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("batch", [1, 2, 3, 4])
def test_gemv_split_rows(layout, batch):
    """Batches 3 and 4 (8-wave blocks for byte-split, 4 for K15 here),
    byte-split at batch 2 (8-wave blocks), and K15 at batch 1 when more than
    one weight in 32 escapes (true here: one row is escape-dense), on rows of more than 4 whole tiles
    (an even number) run each row as 2 parts on separate waves whose sums
    meet in LDS: odd row counts (a block with unused waves), an odd tile
    count (whole rows), both escape forms; bit-identical on a second
    launch."""
    for i, (rows, tiles) in enumerate([(5, 12), (7, 6), (1, 8), (3, 10), (9, 16), (4, 7)]):
        cols = 2048 * tiles
        W = synth.random_bits(rows * cols, 950 + i, "normal").reshape(rows, cols)
        W.reshape(-1)[::97] ^= 0x3000
        W[rows // 2] = synth.random_bits(cols, 960 + i, "uniform") & np.uint16(0xBFFF)
        x = synth.vectors(970 + i, batch, cols)
        y, _ = check_gemv(layout, W, x, what=f"split {rows}x{cols}")
        for form in (0, wc.COMPACT):
            h, c = wc.encode(dev16(W.reshape(-1)), layout | form)
            y1 = wc.decode_gemv(h, c, rows, cols, dev16(x))
            y2 = wc.decode_gemv(h, c, rows, cols, dev16(x))
            torch.cuda.synchronize()
            assert np.array_equal(y1.cpu().numpy().view(np.int32), y2.cpu().numpy().view(np.int32))
            assert np.array_equal(y1.cpu().numpy().view(np.int32), y.view(np.int32)), form


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemv_escape_dense(layout):
    # uniform bit patterns: most symbols escape; includes NaN/inf-free subset
    rows, cols = 64, 4096
    # uniform bit patterns with the top exponent bit cleared: |w| < 2, 256
    # distinct sign+exponent symbols, so most weights escape
    w = synth.random_bits(rows * cols, 901, "uniform") & np.uint16(0xBFFF)
    W = w.reshape(rows, cols)
    x = synth.vectors(902, 4, cols)
    h, c = check_roundtrip(layout, W, "escape-dense")
    assert h.n_esc > rows * cols // 2
    check_gemv(layout, W, x, h, c, "escape-dense")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_clustered_escapes_small(layout):
    """A band of escape-dense rows in a tensor small enough to run as one
    round of waves: every wave of the band starts from an escape-index entry
    that lies deep in the record stream."""
    rows, cols = 1024, 4096
    w = synth.random_bits(rows * cols, 903, "normal").reshape(rows, cols)
    band = synth.random_bits(96 * cols, 904, "uniform").reshape(96, cols) & np.uint16(0xBFFF)
    w[700:796] = band
    x = synth.vectors(905, 4, cols)
    h, c = check_roundtrip(layout, w, "clustered escapes")
    # most escapes are in the band
    d, nd, _ = oracle.dictionary(layout, oracle.histogram(layout, w), w.size)
    sym = w >> (7 if layout == wc.K15 else 8)
    esc = ~np.isin(sym, d[:nd])
    assert esc[700:796].sum() > 0.8 * esc.sum() and h.n_esc == esc.sum()
    check_gemv(layout, w, x, h, c, "clustered escapes")
    check_gemv(layout, w, x[:1], h, c, "clustered escapes, batch 1")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("form", [0, wc.COMPACT], ids=["full", "compact"])
def test_gemv_runs_ahead(layout, form):
    """Tiles whose symbol run comes with their ring loads (every tile of the
    compact form; byte-split full-form tiles that the index shows dense), in
    both slot sizes of the ring kernel: 4104 x 16384 (more than one round of
    waves, 8 tiles per row) takes the large slots at batch 1 and the small
    ones at batches 2 and 4.  Rows hold 0 to 2048 escapes per tile: graded
    counts, rows where every weight escapes (runs longer than a slot holds
    ahead, starting on and off 16-byte boundaries), and uniform rows."""
    rows, cols = 4104, 16384
    rng = np.random.default_rng(991)
    W = synth.random_bits(rows * cols, 990, "normal").reshape(rows, cols)
    hi = synth.BAND_HIGH_BYTES

    def outliers(n):
        return (hi[rng.integers(0, hi.size, n)] << 8) | rng.integers(0, 256, n).astype(np.uint16)

    W[1::16] = synth.random_bits(W[1::16].size, 993, "uniform").reshape(-1, cols) & np.uint16(0xBFFF)
    W[5::512] = outliers(W[5::512].size).reshape(-1, cols)  # too rare for the dictionary
    counts = np.array([0, 30, 65, 200, 520, 1000, 1500, 2040])
    for r in range(3, rows, 8):
        for t, k in enumerate(rng.permutation(counts)):
            W[r, t * 2048 + rng.choice(2048, k, replace=False)] = outliers(k)
    x = synth.vectors(992, 4, cols)
    ref = oracle_gemv(W, x)
    h, c = wc.encode(dev16(W.reshape(-1)), layout | form)
    dec = host16(wc.decode(h, c))
    assert np.array_equal(dec, W.reshape(-1)), "decode"
    for batch in (1, 2, 4):
        check_gemv(layout, W, x[:batch], h, c, f"runs ahead form={form} b={batch}", ref=ref)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gemv_every_batch(layout):
    """Batches 1..16 on shapes with a ragged 16-row block and a partial last
    128-column chunk, and on rows of whole 2048-weight tiles (the LDS-ring
    kernel); escapes in the tensor's last weights (the symbol window of the
    last lanes meets the end of the stream) and one dense band.  Rows of 12
    whole tiles (24576 columns) with a dense band (over 1 weight in 32
    escapes) take the matrix-core kernel's contiguous per-wave ranges at
    batches 8-16."""
    for rows, cols, dense in ((19, 160, False), (45, 1056, True), (13, 4096, True),
                              (21, 24576, True)):
        W = synth.random_bits(rows * cols, 1200 + rows, "normal").reshape(rows, cols)
        flat = W.reshape(-1)
        flat[::211] ^= 0x3000
        flat[-5:] ^= 0x4000
        if dense:
            band = slice(17, 33) if rows > 33 else slice(5, 9)
            nb = band.stop - band.start
            W[band] = synth.random_bits(nb * cols, 1300, "uniform").reshape(nb, cols) & np.uint16(0xBFFF)
        h, c = gpu_encode(layout, W)
        assert h.n_esc > 0
        X = synth.vectors(1400 + rows, 16, cols)
        ref = oracle_gemv(W, X)
        for batch in range(1, 17):
            check_gemv(layout, W, X[:batch], h, c, f"{rows}x{cols} b={batch}", ref=ref)


# --------------------------------------------------- maximum sizes

def _gpu_normal_bits(n: int, seed: int, sigma: float = 0.02) -> torch.Tensor:
    """n BF16 bit patterns of N(0, sigma), drawn on the device from a seeded
    generator (a 2^32-weight tensor is 8 GiB: drawing it on the host would
    take minutes), in 2^28-weight chunks; torch rounds fp32 to BF16 to
    nearest even."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    out = torch.empty(n, dtype=torch.int16, device=DEV)
    step = 1 << 28
    for a in range(0, n, step):
        b = min(n, a + step)
        z = torch.randn(b - a, generator=g, device=DEV, dtype=torch.float32) * sigma
        out[a:b] = z.to(torch.bfloat16).view(torch.int16)
    return out


def _device_counts(w: torch.Tensor, shift: int) -> np.ndarray:
    """Symbol counts of w (b >> shift), counted on the device in chunks."""
    nsym = 1 << (16 - shift)
    counts = torch.zeros(nsym, dtype=torch.int64, device=DEV)
    step = 1 << 28
    for a in range(0, w.numel(), step):
        sym = (w[a:a + step].to(torch.int32) & 0xFFFF) >> shift
        counts += torch.bincount(sym, minlength=nsym)
    return counts.cpu().numpy().astype(np.uint64)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_maximum_size_roundtrip(layout):
    """n = 2^32 - 1, the largest tensor the format holds (u32 positions): the
    last tile is partial and the last code byte holds one nibble; escape
    positions run up to the top of the u32 range.  Checks: exact round trip,
    and the dictionary and escape count equal the oracle's ranking of the
    symbol counts (counted on the device, ranked by the oracle)."""
    n = (1 << 32) - 1
    print(f"max-size round trip: layout={layout} n={n}", flush=True)
    w = _gpu_normal_bits(n, 2024 + layout)
    h, c = wc.encode(w, layout)
    counts = _device_counts(w, 7 if layout == wc.K15 else 8)
    d, nd, ne = oracle.dictionary(layout, counts, n)
    assert (h.n, h.n_dict, h.n_esc) == (n, nd, ne)
    assert list(h.dict)[:nd] == list(d[:nd])
    assert h.total_bytes == oracle.container_size(layout, n, ne)
    del counts
    out = wc.decode(h, c)
    torch.cuda.synchronize()
    assert torch.equal(out, w), "maximum-size tensor not rebuilt exactly"
    # the last escape records sit near the top of the position range
    last_pos = int(c[h.off_esc_pos + 4 * (h.n_esc - 1):h.off_esc_pos + 4 * h.n_esc].cpu().numpy().view("<u4")[0])
    assert last_pos > n - (1 << 20)


def test_maximum_size_gemv():
    """65535 x 65536 (n just below 2^32), byte-split, batch 1 (LDS-ring
    kernel), 16 (matrix cores) and 64 (wide matrix-core kernel): sampled rows
    against the oracle."""
    rows, cols = 65535, 65536
    print(f"max-size GEMV: {rows}x{cols}", flush=True)
    w = _gpu_normal_bits(rows * cols, 2030)
    h, c = wc.encode(w, wc.BYTESPLIT)
    X = synth.vectors(2031, 64, cols)
    sample = [0, 1, 2047, 32768, rows - 2, rows - 1]
    Ws = w.view(rows, cols)[sample].cpu().numpy().view(np.uint16)
    for batch in (1, 16, 64):
        print(f"max-size GEMV batch {batch}", flush=True)
        y = wc.decode_gemv(h, c, rows, cols, dev16(X[:batch]))
        torch.cuda.synchronize()
        y64, a = oracle.gemv_f64(Ws, X[:batch])
        assert_gemv_close(y.cpu().numpy()[:, sample], y64, a, f"max-size GEMV b={batch}")


# ------------------------------------------- raw layout and layout choice

@pytest.mark.parametrize("kind", ["normal", "uniform"])
def test_raw_layout_roundtrip(kind):
    for i, n in enumerate([1, 7, 8, 9, 2047, 2049, 65537, (1 << 20) + 3]):
        h, _ = check_roundtrip(wc.RAW, synth.random_bits(n, 1500 + i, kind), f"raw {kind} n={n}")
        assert (h.layout, h.n_dict, h.n_esc) == (wc.RAW, 0, 0)


def test_raw_layout_gemv():
    for i, (rows, cols, batch) in enumerate([(33, 4096, 1), (17, 100, 3), (64, 2048, 16), (9, 6144, 8)]):
        W = synth.random_bits(rows * cols, 1600 + i, "uniform").reshape(rows, cols) & np.uint16(0xBFFF)
        x = synth.vectors(1700 + i, batch, cols)
        check_gemv(wc.RAW, W, x, what=f"raw {rows}x{cols} b={batch}")


def test_auto_layout_matches_oracle_choice():
    """wc_build_dict with WC_LAYOUT_AUTO picks the layout the oracle picks
    (smallest container, ties to the lower number), and encodes it byte for
    byte as the oracle does."""
    from tests.test_oracle import _choice_cases
    cases = [(name, w) for name, w, _ in _choice_cases()]
    cases.append(("mlp W1", synth.mlp()["W1"].reshape(-1)))
    cases.append(("banded", synth.banded()["W"].reshape(-1)))
    for name, w in cases:
        want = oracle.choose_layout(w)
        h, c = gpu_encode(wc.AUTO, w)
        assert h.layout == want, (name, h.layout, want)
        assert np.array_equal(c.cpu().numpy(), oracle.encode(want, w)), name
        if w.size:
            out = wc.decode(h, c)
            torch.cuda.synchronize()
            assert np.array_equal(host16(out), w), name


def test_artifact_streamed_verify(tmp_path):
    """Tensors encoded on the GPU, written to an artifact, then streamed back:
    read (every CRC checked), uploaded, decoded exactly, and the decoded
    values' CRC-32 equal to the source's."""
    import zlib
    tensors = [("small", synth.small()["W"]), ("square", synth.square()["W"]),
               ("layer.norm", synth.layerset_tensor(72)[1]),
               ("uniform", synth.random_bits(64 * 4096, 1800, "uniform").reshape(64, 4096))]
    items, sources = [], {}
    for name, W in tensors:
        h, c = gpu_encode(wc.AUTO, W)
        items.append((name, W.shape, c, zlib.crc32(np.ascontiguousarray(W).tobytes())))
        sources[name] = (W, h.layout)
    path = str(tmp_path / "set.wca")
    wc.artifact_write(path, items)
    res = wc.artifact_verify(path, DEV)
    assert [r[0] for r in res] == [t[0] for t in tensors]
    assert all(r[1] for r in res), res
    for i, e in enumerate(wc.artifact_entries(path)):
        W, lay = sources[e["name"]]
        assert e["layout"] == lay
        c = torch.from_numpy(wc.artifact_read(path, i)).to(DEV)
        out = wc.decode(wc.read_header(c), c)
        torch.cuda.synchronize()
        assert np.array_equal(host16(out), np.ascontiguousarray(W).reshape(-1)), e["name"]


def test_gemv_cols_zero_and_rows_zero():
    w = torch.empty(0, dtype=torch.int16, device=DEV)
    h, c = wc.encode(w, wc.BYTESPLIT)
    x = torch.zeros((3, 0), dtype=torch.int16, device=DEV)
    y = torch.full((3, 5), 7.0, device=DEV)
    wc.decode_gemv(h, c, 5, 0, x, out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
    y0 = torch.empty((3, 0), device=DEV)
    wc.decode_gemv(h, c, 0, 17, torch.zeros((3, 17), dtype=torch.int16, device=DEV), out=y0)
    # the same at a batch for the wide path
    y = torch.full((64, 5), 7.0, device=DEV)
    wc.decode_gemv(h, c, 5, 0, torch.zeros((64, 0), dtype=torch.int16, device=DEV), out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)
    wc.decode_gemv(h, c, 0, 128, torch.zeros((64, 128), dtype=torch.int16, device=DEV),
                   out=torch.empty((64, 0), device=DEV))


def test_error_codes():
    """The library's own status codes, called through the C ABI directly (the
    binding rejects these arguments itself before any library call)."""
    import ctypes
    W = synth.random_bits(64 * 64, 1, "normal").reshape(64, 64)
    h, c = gpu_encode(0, W)
    lib = wc._lib
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    x = dev16(synth.vectors(1, 257, 64))
    y = torch.empty((257, 64), dtype=torch.float32, device=DEV)
    assert lib.wc_decode_gemv(ctypes.byref(h), P(c.data_ptr()), c.numel(), 64, 64,
                              P(x.data_ptr()), 257, P(y.data_ptr()), s) == -5
    assert lib.wc_decode_gemv(ctypes.byref(h), P(c.data_ptr()), c.numel(), 32, 64,
                              P(x.data_ptr()), 1, P(y.data_ptr()), s) == -1
    bad = wc.Header.from_bytes(h.to_bytes())
    bad.n_esc = bad.n + 1
    out = torch.empty(h.n, dtype=torch.int16, device=DEV)
    assert lib.wc_decode(ctypes.byref(bad), P(c.data_ptr()), c.numel(), P(out.data_ptr()), s) == -3
    assert lib.wc_decode(ctypes.byref(h), P(c.data_ptr()), h.total_bytes - 16,
                         P(out.data_ptr()), s) == -2
    # misaligned output
    buf = torch.empty(h.n + 8, dtype=torch.int16, device=DEV)
    with pytest.raises(wc.WCError) as e:
        wc.decode(h, c, out=buf[1:1 + h.n])
    assert e.value.code == -1
    # the binding's own checks come first
    with pytest.raises(ValueError):
        wc.decode_gemv(h, c, 64, 64, x)
    with pytest.raises(ValueError):
        wc.decode(h, c[: h.total_bytes - 16])
    torch.cuda.synchronize()


def test_determinism():
    d = synth.square()
    W = d["W"]
    for layout in LAYOUTS:
        h1, c1 = gpu_encode(layout, W)
        h2, c2 = gpu_encode(layout, W)
        assert torch.equal(c1, c2)
        x = dev16(synth.vectors(2, 4, 4096))
        y1 = wc.decode_gemv(h1, c1, 4096, 4096, x)
        y2 = wc.decode_gemv(h1, c1, 4096, 4096, x)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


# --------------------------------------------------- the five workloads

def test_workload_small():
    d = synth.small()
    h, c = check_roundtrip(wc.BYTESPLIT, d["W"], "small byte-split")
    check_gemv(wc.BYTESPLIT, d["W"], d["x"], h, c, "small byte-split")
    h, c = check_roundtrip(wc.K15, d["W"], "small K15")
    check_gemv(wc.K15, d["W"], d["x"], h, c, "small K15")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_workload_square(layout):
    d = synth.square()
    h, c = check_roundtrip(layout, d["W"], "square")
    check_gemv(layout, d["W"], d["x"], h, c, "square")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_workload_mlp(layout):
    m = synth.mlp()
    for name, xn in (("W1", "x1"), ("W2", "x2")):
        h, c = check_roundtrip(layout, m[name], f"mlp {name}")
        check_gemv(layout, m[name], m[xn], h, c, f"mlp {name}")


@pytest.mark.parametrize("t", [0, 47, 48, 71, 72, 95])
def test_workload_layerset_tensors(t):
    name, a = synth.layerset_tensor(t)
    for layout in LAYOUTS:
        check_roundtrip(layout, a, f"layerset {name}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("t", [0, 48])
def test_gemv_layerset_sampled(layout, t):
    """The layer set's 6144 x 24576 and 24576 x 6144 tensors (drawn on the
    GPU) at batches 1, 3, 4 and 16: byte-split at batch 4 takes the matrix
    cores on grids this large (fewer than one weight in 64 escapes), K15
    the LDS ring (at batches 3 and 4 the 6144 x 24576 rows split in two, in
    blocks of 8 waves); 256 sampled rows against the oracle."""
    _, (rows, cols), w = synth.layerset_tensor_device(t, DEV)
    h, c = wc.encode(w, layout)
    X = synth.vectors(2800 + t, 16, cols)
    sample = np.sort(np.random.default_rng(11 + t).choice(rows, 256, replace=False))
    Ws = w.view(rows, cols)[torch.from_numpy(sample).to(DEV)].cpu().numpy().view(np.uint16)
    y64, a = oracle.gemv_f64(np.ascontiguousarray(Ws), X)
    for batch in (1, 3, 4, 16):
        y = wc.decode_gemv(h, c, rows, cols, dev16(X[:batch]))
        torch.cuda.synchronize()
        assert_gemv_close(y.cpu().numpy()[:, sample], y64[:batch], a[:batch],
                          f"layerset {t} layout {layout} b={batch}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_workload_banded(layout):
    d = synth.banded()
    W = d["W"]
    h, c = check_roundtrip(layout, W, "banded")
    ref = oracle_gemv(W, d["X"])
    for batch in (1, 4, 16):
        check_gemv(layout, W, d["X"][:batch], h, c, f"banded b={batch}", ref=ref)
