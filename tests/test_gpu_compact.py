"""GPU parity of the compact escape form (header flag WC_FLAG_COMPACT: the
escape stream holds the symbols only, the k-th code-15 weight takes the k-th
symbol): containers byte-identical to the oracle's compact containers, and
exact decode and the fused GEMV on every kernel path, every tile with
escapes placing its symbols by in-wave rank and rows that start inside an
index tile counting the code-15 marks from the tile start."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_gemv_sign_amd as wc  # noqa: E402
from tests.test_gpu_parity import dev16, host16  # noqa: E402
from tests.tolerance import assert_gemv_close  # noqa: E402

LAYOUTS = [wc.BYTESPLIT, wc.K15]


def check_compact(layout, w_np, what):
    w_flat = np.ascontiguousarray(w_np).reshape(-1)
    h, c = wc.encode(dev16(w_flat), layout | wc.COMPACT)
    torch.cuda.synchronize()
    assert h.flags == (wc.FLAG_COMPACT if layout != wc.RAW else 0), what
    ref = oracle.encode(layout, w_flat, oracle.COMPACT if layout != wc.RAW else 0)
    got = c.cpu().numpy()
    assert got.size == ref.size, f"{what}: size {got.size} vs {ref.size}"
    if not np.array_equal(got, ref):
        bad = np.nonzero(got != ref)[0]
        raise AssertionError(f"{what}: {bad.size} bytes differ, first at {bad[0]}")
    out = wc.decode(h, c)
    torch.cuda.synchronize()
    assert np.array_equal(host16(out), w_flat), f"{what}: decode not exact"
    return h, c


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compact_bit_patterns_and_ragged(layout):
    check_compact(layout, synth.all_patterns(11), "all bit patterns")
    for n in (1, 7, 2047, 2048, 2049, 8191, 8193, 100003):
        for kind in ("normal", "uniform"):
            check_compact(layout, synth.random_bits(n, 3000 + n, kind), f"n={n} {kind}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compact_workloads(layout):
    """The square tensor (sparse escapes), the banded one (dense bands) and
    the MLP pair (K15: 28% escapes)."""
    check_compact(layout, synth.square()["W"], "square")
    check_compact(layout, synth.banded()["W"], "banded")
    m = synth.mlp()
    check_compact(layout, m["W1"], "mlp W1")


def test_compact_auto_and_raw():
    w = synth.random_bits(50000, 3100, "normal")
    h, c = wc.encode(dev16(w), wc.AUTO | wc.COMPACT)
    torch.cuda.synchronize()
    assert h.flags == wc.FLAG_COMPACT
    assert np.array_equal(host16(wc.decode(h, c)), w)
    check_compact(wc.RAW, synth.random_bits(1000, 3101, "uniform"), "raw")


def _tensor(rows, cols, dense, seed):
    W = synth.random_bits(rows * cols, seed, "normal").reshape(rows, cols)
    flat = W.reshape(-1)
    flat[::211] ^= 0x3000
    flat[-5:] ^= 0x4000
    if dense:
        band = slice(17, 33) if rows > 33 else slice(5, 9)
        nb = band.stop - band.start
        W[band] = synth.random_bits(nb * cols, seed + 1, "uniform").reshape(nb, cols) & np.uint16(0xBFFF)
    return W


# (rows, cols, dense escapes, batches): rows inside index tiles (cursor by
# counting code-15 marks), whole-tile rows (LDS ring), cols % 8 != 0
# (generic kernel), 12-tile rows with a dense band (contiguous matrix-core
# ranges), and wide batches with and without column splits
GEMV_CASES = [
    (19, 160, False, (1, 4, 8, 16)),
    (45, 1056, True, (1, 3, 8, 16, 40)),
    (13, 4096, True, (1, 2, 4, 16, 64)),
    (7, 100, False, (1, 5)),
    (21, 24576, True, (1, 8, 16)),
    (77, 640, True, (64,)),
    (130, 4096, True, (100, 256)),
]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("rows,cols,dense,batches", GEMV_CASES,
                         ids=[f"{r}x{c}" for r, c, _, _ in GEMV_CASES])
def test_compact_gemv(layout, rows, cols, dense, batches):
    """The fused product on compact containers equals the oracle's sums on
    the same weights, on every kernel path."""
    W = _tensor(rows, cols, dense, 3300 + rows)
    h, c = check_compact(layout, W, f"{rows}x{cols}")
    assert h.n_esc > 0
    X = synth.vectors(3400 + rows, max(batches), cols)
    y32 = oracle.gemv_f32(W, X)
    y64, a = oracle.gemv_f64(W, X)
    for batch in batches:
        y = wc.decode_gemv(h, c, rows, cols, dev16(X[:batch]))
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        what = f"compact {rows}x{cols} layout {layout} b={batch}"
        assert_gemv_close(y, y32[:batch], a[:batch], what + " vs fp32")
        assert_gemv_close(y, y64[:batch], a[:batch], what + " vs fp64")


def test_compact_gemv_banded_sampled():
    """6144 x 24576 banded tensor, K15 compact, batches 1, 16 and 64; 256
    sampled rows."""
    W = synth.banded()["W"]
    rows, cols = W.shape
    h, c = check_compact(wc.K15, W, "banded")
    X = synth.vectors(3500, 64, cols)
    sample = np.sort(np.random.default_rng(10).choice(rows, 256, replace=False))
    y64, a = oracle.gemv_f64(np.ascontiguousarray(W[sample]), X)
    for batch in (1, 16, 64):
        y = wc.decode_gemv(h, c, rows, cols, dev16(X[:batch]))
        torch.cuda.synchronize()
        assert_gemv_close(y.cpu().numpy()[:, sample], y64[:batch], a[:batch],
                          f"banded compact b={batch}")
