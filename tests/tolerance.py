"""Acceptance rule for GEMV outputs.

Exact weights do not fix the output once the accumulation order changes
(page "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está listo
para producción?", section "¿Qué significa “sin pérdida” para los pesos de
un LLM?").  The required bound is a relative error of 1e-3 per output
element.  Products of BF16 values are exact in fp32, so two valid fp32
summation orders differ by at most about cols * 2^-24 * a, where
a = sum_c |W[r,c] x[c]|; when the sum cancels (|y| much smaller than a)
that difference is no longer small relative to |y|.  An element therefore
passes when |y - y_ref| <= 1e-3 * max(|y_ref|, 2^-10 * a): the plain relative
bound wherever |y_ref| >= 2^-10 a, and an absolute floor of about 1e-6 a
for outputs that cancel below that.
"""
import numpy as np

REL = 1e-3
FLOOR = 2.0 ** -10


def gemv_excess(y, y_ref, a):
    """Per-element |y - y_ref| / bound; an element passes when <= 1."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    bound = REL * np.maximum(np.abs(y_ref), FLOOR * a)
    err = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return r


def assert_gemv_close(y, y_ref, a, what=""):
    r = gemv_excess(y, y_ref, a)
    bad = np.argwhere(~(r <= 1.0))
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {bad.shape[0]} of {r.size} outputs out of tolerance; first at {i}: "
            f"y={np.asarray(y)[i]!r} ref={np.asarray(y_ref)[i]!r} a={np.asarray(a)[i]!r}")
