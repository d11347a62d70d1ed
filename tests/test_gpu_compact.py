"""GPU parity of the compact escape form (header flag WC_FLAG_COMPACT: the
escape stream holds the symbols only, the k-th code-15 weight takes the k-th
symbol): containers byte-identical to the oracle's compact containers, and
exact decode, every tile with escapes placing its symbols by in-wave rank.
The fused GEMV does not take this form yet and must refuse it."""
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


def test_compact_gemv_refused():
    W = synth.random_bits(64 * 256, 3200, "normal").reshape(64, 256)
    h, c = wc.encode(dev16(W), wc.K15 | wc.COMPACT)
    with pytest.raises(wc.WCError) as e:
        wc.decode_gemv(h, c, 64, 256, dev16(synth.vectors(3201, 1, 256)))
    assert e.value.code == -5
