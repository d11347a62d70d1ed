"""GPU parity above 16 input rows (the wide matrix-core path from batch 33,
or 17 on tensors of 2^26 weights or more; smaller batches run 16 rows at a
time): the fused decode-GEMM and the plain BF16 kernel of the same shape
against the CPU oracle, to the same per-element bar as the GEMV
(tests/tolerance.py).

This is the prefill regime, where page "Compresión de pesos LLM sin pérdida
vs 8-bit GGUF: ¿qué está listo para producción?", section "¿Cómo encaja con
los sistemas anteriores?", names a fused decompression-GEMM as the closest
prior design.  Cases: one and several 128-column chunks, rows that fill no
whole 16-row tile, rows on and off the 2048-weight escape-index grid (index
load vs search), a dense escape band, batch groups with a partial last
tile, and a column count that is no multiple of 128 (16 rows at a time).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.tolerance import assert_gemv_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_gemv_sign_amd as wc  # noqa: E402
from tests.test_gpu_parity import DEV, dev16, gpu_encode, oracle_gemv  # noqa: E402

LAYOUTS = [wc.BYTESPLIT, wc.K15]
BATCHES = (17, 31, 32, 33, 64, 65, 100, 256)


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


@pytest.mark.parametrize("layout", LAYOUTS + [wc.RAW])
@pytest.mark.parametrize("rows,cols,dense", [(1, 4096, False), (19, 128, False), (77, 640, True),
                                             (130, 4096, True), (45, 1056, True)])
def test_wide_batches(layout, rows, cols, dense):
    W = _tensor(rows, cols, dense, 2100 + rows)
    h, c = gpu_encode(layout, W)
    if layout != wc.RAW:
        assert h.n_esc > 0
    X = synth.vectors(2200 + rows, max(BATCHES), cols)
    y32, y64, a = oracle_gemv(W, X)
    Wd = dev16(W)
    for batch in BATCHES:
        xd = dev16(X[:batch])
        y = wc.decode_gemv(h, c, rows, cols, xd)
        yb = wc.gemv_bf16(Wd, xd)
        torch.cuda.synchronize()
        what = f"{rows}x{cols} layout {layout} b={batch}"
        y = y.cpu().numpy()
        assert_gemv_close(y, y32[:batch], a[:batch], f"{what} fused vs oracle fp32")
        assert_gemv_close(y, y64[:batch], a[:batch], f"{what} fused vs oracle fp64")
        assert_gemv_close(yb.cpu().numpy(), y64[:batch], a[:batch], f"{what} plain vs oracle fp64")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_wide_square_workload_sampled(layout):
    """4096 x 4096 square workload at batch 64 and 256, as the benchmark
    runs it; 512 sampled rows are compared (the oracle computes each output
    on its own)."""
    d = synth.square()
    W = d["W"]
    rows, cols = W.shape
    h, c = gpu_encode(layout, W)
    X = synth.vectors(synth.SEEDS["square"] * 10 + 7, 256, cols)
    sample = np.sort(np.random.default_rng(7).choice(rows, 512, replace=False))
    y64, a = oracle.gemv_f64(np.ascontiguousarray(W[sample]), X)
    for batch in (64, 256):
        y = wc.decode_gemv(h, c, rows, cols, dev16(X[:batch]))
        torch.cuda.synchronize()
        assert_gemv_close(y.cpu().numpy()[:, sample], y64[:batch], a[:batch],
                          f"square b={batch}")


def test_wide_banded_sampled():
    """6144 x 24576 with 5% escapes in 64-row bands (rows of 12 index
    tiles), K15, byte-split and the plain kernel, batches 24 (a tensor this
    large takes the wide kernel from batch 17) and 64; 384 sampled rows."""
    d = synth.banded()
    W = d["W"]
    rows, cols = W.shape
    X = synth.vectors(synth.SEEDS["banded"] * 10 + 7, 64, cols)
    sample = np.sort(np.random.default_rng(8).choice(rows, 384, replace=False))
    y64, a = oracle.gemv_f64(np.ascontiguousarray(W[sample]), X)
    Wd = dev16(W)
    for batch in (24, 64):
        xd = dev16(X[:batch])
        yb = wc.gemv_bf16(Wd, xd)
        torch.cuda.synchronize()
        assert_gemv_close(yb.cpu().numpy()[:, sample], y64[:batch], a[:batch],
                          f"banded plain b={batch}")
        for layout in LAYOUTS:
            h, c = gpu_encode(layout, W)
            y = wc.decode_gemv(h, c, rows, cols, xd)
            torch.cuda.synchronize()
            assert_gemv_close(y.cpu().numpy()[:, sample], y64[:batch], a[:batch],
                              f"banded layout {layout} b={batch}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_wide_tall_sampled(layout):
    """24576 x 6144 N(0, 0.015) (a tall tensor of the layer set, drawn on the
    GPU): at batches up to 64 a tensor this large takes two batch tiles per
    block, with 2 waves per block at batch 32 and 4 at batches 48 and 64 (two
    batch groups); 256 sampled rows against the oracle."""
    _, (rows, cols), w = synth.layerset_tensor_device(48, DEV)
    h, c = wc.encode(w, layout)
    X = synth.vectors(2700, 64, cols)
    sample = np.sort(np.random.default_rng(10).choice(rows, 256, replace=False))
    Ws = w.view(rows, cols)[torch.from_numpy(sample).to(DEV)].cpu().numpy().view(np.uint16)
    y64, a = oracle.gemv_f64(np.ascontiguousarray(Ws), X)
    for batch in (32, 48, 64):
        y = wc.decode_gemv(h, c, rows, cols, dev16(X[:batch]))
        torch.cuda.synchronize()
        assert_gemv_close(y.cpu().numpy()[:, sample], y64[:batch], a[:batch],
                          f"tall layout {layout} b={batch}")


def test_wide_deterministic():
    W = _tensor(130, 4096, True, 2300)
    h, c = gpu_encode(wc.K15, W)
    xd = dev16(synth.vectors(2301, 100, 4096))
    y1 = wc.decode_gemv(h, c, 130, 4096, xd)
    y2 = wc.decode_gemv(h, c, 130, 4096, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_wide_mlp_sampled(layout):
    """The MLP pair (14336 x 4096 and 4096 x 14336, row scales over three
    decades: K15 escapes about 28% of the weights, so nearly every lane patches
    its symbols every step), batch 64 and 100; 256 sampled rows each."""
    m = synth.mlp()
    for name in ("W1", "W2"):
        W = m[name]
        rows, cols = W.shape
        h, c = gpu_encode(layout, W)
        X = synth.vectors(synth.SEEDS["mlp"] * 10 + 7, 100, cols)
        sample = np.sort(np.random.default_rng(9).choice(rows, 256, replace=False))
        y64, a = oracle.gemv_f64(np.ascontiguousarray(W[sample]), X)
        for batch in (64, 100):
            y = wc.decode_gemv(h, c, rows, cols, dev16(X[:batch]))
            torch.cuda.synchronize()
            assert_gemv_close(y.cpu().numpy()[:, sample], y64[:batch], a[:batch],
                              f"mlp {name} layout {layout} b={batch}")


def test_wide_random_shapes():
    """Seeded random shapes: rows 1..300, columns a multiple of 128 (on and
    off the 2048-weight index grid) or not, batches 17..256, both layouts,
    escape densities from sparse to dense rows."""
    rng = np.random.default_rng(2400)
    for case in range(16):
        rows = int(rng.integers(1, 301))
        k = int(rng.integers(1, 33))
        cols = 128 * k if case % 4 else 128 * k + 32
        batch = int(rng.integers(17, 257))
        layout = LAYOUTS[case % 2]
        W = _tensor(rows, cols, bool(case % 3 == 0), 2500 + case)
        X = synth.vectors(2600 + case, batch, cols)
        h, c = gpu_encode(layout, W)
        y = wc.decode_gemv(h, c, rows, cols, dev16(X))
        torch.cuda.synchronize()
        y64, a = oracle.gemv_f64(W, X)
        assert_gemv_close(y.cpu().numpy(), y64, a,
                          f"case {case}: {rows}x{cols} layout {layout} b={batch}")
