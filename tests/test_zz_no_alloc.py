"""wc_encode_noalloc: the encode entry point that allocates nothing, for
callers that cannot allocate device memory (graph capture, serving loops).
Its containers must equal wc_encode's byte for byte, on consecutive calls
that share the library's one scratch array, the second with a smaller
tensor (the array keeps the first call's state, which every call clears
before use)."""
import ctypes

import numpy as np
import pytest

import synth

gpu = pytest.mark.gpu


def _lib():
    import decode_gemv_sign_amd as wc
    return wc


def _noalloc_header(n: int):
    """A valid byte-split header of n weights without escapes (host only)."""
    wc = _lib()
    h = wc.Header()
    h.magic = 0x36314357
    h.version = 2
    h.layout = 0
    h.n = n
    pad = lambda x: (x + 15) // 16 * 16  # noqa: E731
    h.off_codes = 128
    h.off_raw = pad(128 + (n + 1) // 2)
    h.off_esc_pos = pad(h.off_raw + n)
    h.off_esc_sym = h.off_esc_pos
    h.off_esc_idx = h.off_esc_sym
    h.total_bytes = h.off_esc_idx
    return h


def test_noalloc_rejects_tensors_beyond_its_scratch():
    """n above WC_NOALLOC_MAX_N (2^31) is refused before any device work."""
    wc = _lib()
    h = _noalloc_header((1 << 31) + 8)
    P = ctypes.c_void_p
    assert wc._lib.wc_encode_noalloc(ctypes.byref(h), P(16), P(16), h.total_bytes, None) == -2
    h = _noalloc_header(1 << 31)
    # at the limit the size check passes; a misaligned container is refused next
    assert wc._lib.wc_encode_noalloc(ctypes.byref(h), P(16), P(8), h.total_bytes, None) == -1


@gpu
@pytest.mark.parametrize("layout", [0, 1])
def test_noalloc_matches_encode_on_consecutive_calls(layout):
    import torch
    wc = _lib()
    dev = "cuda:0"
    big = synth.square()["W"]                      # 16.8M weights, escapes in most tiles
    small = synth.banded(rows=256, cols=4096, bands=1)["W"]  # 1M weights, one dense escape band
    for W in (big, small):
        w = torch.from_numpy(np.ascontiguousarray(W).reshape(-1).view(np.int16)).to(dev)
        h = wc.build_dict(w, layout)
        ref = torch.empty(h.total_bytes, dtype=torch.uint8, device=dev)
        wc.encode_into(h, w, ref)
        got = torch.full((h.total_bytes,), 0xA5, dtype=torch.uint8, device=dev)
        wc.encode_into_noalloc(h, w, got)
        torch.cuda.synchronize()
        assert h.n_esc > 0
        assert torch.equal(got, ref), (layout, W.shape)
        # and the decode of the no-alloc container is exact
        out = wc.decode(h, got)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), np.ascontiguousarray(W).reshape(-1))
