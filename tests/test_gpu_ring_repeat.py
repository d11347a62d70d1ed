"""Bounded repeat test of the kernels that stream tiles through an LDS ring
filled by global->LDS loads (decode and the fused GEMV at batches 1 and 4).

Their waits count only global->LDS loads and take those to complete in
issue order among themselves (the rule the compiler's own wait placement
uses for one kind of vector-memory operation).  A wait that relied on
anything else would show as an output that changes from launch to launch:
once, a GEMV that counted ordinary loads in its wait gave one wrong row in
4096 now and then, on a shape with one row per wave.  Each case here is
launched REPEATS times into separate buffers and every output is compared
bit for bit with the first launch, which is itself checked against the
oracle; the test stops at the first mismatch."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import decode_gemv_sign_amd as wc  # noqa: E402
from tests.test_gpu_parity import dev16  # noqa: E402
from tests.tolerance import assert_gemv_close  # noqa: E402

REPEATS = 64
BUFS = 8


def _repeat_equal(launch, ref, what):
    outs = [torch.empty_like(ref) for _ in range(BUFS)]
    for rep in range(REPEATS):
        launch(outs[rep % BUFS])
        if rep % BUFS == BUFS - 1:
            torch.cuda.synchronize()
            for k, o in enumerate(outs):
                if not torch.equal(o.view(torch.int32) if o.dtype == torch.float32 else o,
                                   ref.view(torch.int32) if ref.dtype == torch.float32 else ref):
                    bad = torch.nonzero((o != ref).reshape(-1))[:4, 0].cpu().tolist()
                    raise AssertionError(f"{what}: launch {rep - BUFS + 1 + k} differs from the "
                                         f"first at flat indices {bad}")


@pytest.mark.parametrize("form", [0, wc.COMPACT], ids=["full", "compact"])
@pytest.mark.parametrize("layout", [wc.BYTESPLIT, wc.K15], ids=["bs", "k15"])
def test_square_one_row_per_wave(layout, form):
    """4096 x 4096: the fused GEMV runs one row (two ring tiles) per wave."""
    W = synth.square()["W"]
    rows, cols = W.shape
    w = dev16(W.reshape(-1))
    h, c = wc.encode(w, layout | form)
    for B in (1, 4):
        X = synth.vectors(2, B, cols)
        x = dev16(X)
        y0 = wc.decode_gemv(h, c, rows, cols, x)
        torch.cuda.synchronize()
        y64, a = oracle.gemv_f64(W, X)
        assert_gemv_close(y0.cpu().numpy(), y64, a, f"square layout {layout} form {form} B={B}")
        _repeat_equal(lambda o: wc.decode_gemv(h, c, rows, cols, x, out=o), y0,
                      f"fused GEMV layout {layout} form {form} B={B}")
    d0 = wc.decode(h, c)
    torch.cuda.synchronize()
    assert np.array_equal(d0.cpu().numpy().view(np.uint16), W.reshape(-1))
    _repeat_equal(lambda o: wc.decode(h, c, out=o), d0, f"decode layout {layout} form {form}")


@pytest.mark.parametrize("layout", [wc.BYTESPLIT, wc.K15], ids=["bs", "k15"])
def test_banded_rows_of_whole_tiles(layout):
    """6144 x 24576 with dense escape bands: 12 ring tiles per row."""
    d = synth.banded()
    W = d["W"]
    rows, cols = W.shape
    h, c = wc.encode(dev16(W.reshape(-1)), layout)
    X = d["X"][:1]
    x = dev16(X)
    y0 = wc.decode_gemv(h, c, rows, cols, x)
    torch.cuda.synchronize()
    sel = np.r_[0:64, int(d["bands"][0]) * 64:int(d["bands"][0]) * 64 + 64]
    y64, a = oracle.gemv_f64(np.ascontiguousarray(W[sel]), X)
    assert_gemv_close(y0.cpu().numpy()[:, sel], y64, a, f"banded layout {layout}")
    _repeat_equal(lambda o: wc.decode_gemv(h, c, rows, cols, x, out=o), y0,
                  f"banded fused GEMV layout {layout}")
