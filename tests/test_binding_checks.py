"""The binding's argument checks (no GPU).

The C ABI receives bare device pointers for x, y and the decode output, so it
cannot see how large they are: a GEMV called with fewer x rows than its batch
reads past the end of x.  The binding therefore checks every tensor's shape,
dtype, layout and device before it calls the library.  Each case below must
raise before any library call: the library is replaced by a stub that records
calls, and the tensors live on PyTorch's "meta" device (shapes without
memory), which the test lets stand in for device memory."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import decode_gemv_sign_amd as wc  # noqa: E402


class _StubLib:
    """Stands in for libwc: records calls, returns WC_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        if not name.startswith("wc_"):
            raise AttributeError(name)

        def f(*args):
            self.calls.append(name)
            return 0
        return f


class _Stream:
    cuda_stream = 0


@pytest.fixture
def stub(monkeypatch):
    lib = _StubLib()
    monkeypatch.setattr(wc, "_lib", lib)
    monkeypatch.setattr(wc, "_on_device", lambda t: t.device.type == "meta")
    monkeypatch.setattr(wc, "_ptr", lambda t: None)
    return lib


META = torch.device("meta")


def header(n: int, total: int) -> wc.Header:
    h = wc.Header()
    h.n = n
    h.total_bytes = total
    return h


def t16(*shape, device=META):
    return torch.empty(shape, dtype=torch.int16, device=device)


def f32(*shape, device=META):
    return torch.empty(shape, dtype=torch.float32, device=device)


def u8(n, device=META):
    return torch.empty(n, dtype=torch.uint8, device=device)


ROWS, COLS = 6, 32
H = header(ROWS * COLS, 512)
S = _Stream()


def test_valid_calls_reach_the_library(stub):
    wc.decode_gemv(H, u8(512), ROWS, COLS, t16(4, COLS), out=f32(4, ROWS), stream=S)
    wc.decode_gemv(H, u8(600), ROWS, COLS, t16(COLS), out=f32(ROWS), stream=S)
    wc.gemv_bf16(t16(ROWS, COLS), t16(3, COLS), out=f32(3, ROWS), stream=S)
    wc.decode(H, u8(512), out=t16(ROWS * COLS + 5), stream=S)
    wc.encode_into(H, t16(ROWS * COLS), u8(512), work=u8(wc.workspace_bytes(ROWS * COLS)),
                   stream=S)
    assert stub.calls == ["wc_decode_gemv", "wc_decode_gemv", "wc_gemv_bf16", "wc_decode",
                          "wc_encode"]


@pytest.mark.parametrize("case", [
    "x_fewer_rows_than_out", "x_wrong_cols", "x_3d", "x_batch_too_large", "x_float",
    "out_wrong_rows", "out_wrong_batch", "out_dtype", "out_noncontig", "out_on_host",
    "x_on_host", "container_short", "container_dtype", "container_on_host", "shape_not_n",
])
def test_decode_gemv_rejects(stub, case):
    c, x, out, rows, cols = u8(512), t16(4, COLS), f32(4, ROWS), ROWS, COLS
    if case == "x_fewer_rows_than_out":
        x = t16(1, COLS)  # batch 1 against a 4-row output
    elif case == "x_wrong_cols":
        x = t16(4, COLS - 8)
    elif case == "x_3d":
        x = t16(2, 2, COLS)
    elif case == "x_batch_too_large":
        x, out = t16(257, COLS), f32(257, ROWS)
    elif case == "x_float":
        x = f32(4, COLS)
    elif case == "out_wrong_rows":
        out = f32(4, ROWS - 1)
    elif case == "out_wrong_batch":
        out = f32(2, ROWS)
    elif case == "out_dtype":
        out = t16(4, ROWS)
    elif case == "out_noncontig":
        out = f32(ROWS, 4).t()
    elif case == "out_on_host":
        out = f32(4, ROWS, device="cpu")
    elif case == "x_on_host":
        x = t16(4, COLS, device="cpu")
    elif case == "container_short":
        c = u8(511)
    elif case == "container_dtype":
        c = t16(512)
    elif case == "container_on_host":
        c = u8(512, device="cpu")
    elif case == "shape_not_n":
        rows = ROWS + 1
        out = f32(4, rows)
    with pytest.raises((ValueError, TypeError)):
        wc.decode_gemv(H, c, rows, cols, x, out=out, stream=S)
    assert stub.calls == []


@pytest.mark.parametrize("case", ["x_rows", "x_cols", "out_shape", "out_dtype", "w_1d",
                                  "x_on_host"])
def test_gemv_bf16_rejects(stub, case):
    w, x, out = t16(ROWS, COLS), t16(3, COLS), f32(3, ROWS)
    if case == "x_rows":
        x = t16(2, COLS)
    elif case == "x_cols":
        x = t16(3, COLS + 8)
    elif case == "out_shape":
        out = f32(3, ROWS + 1)
    elif case == "out_dtype":
        out = torch.empty((3, ROWS), dtype=torch.float64, device=META)
    elif case == "w_1d":
        w = t16(ROWS * COLS)
    elif case == "x_on_host":
        x = t16(3, COLS, device="cpu")
    with pytest.raises((ValueError, TypeError)):
        wc.gemv_bf16(w, x, out=out, stream=S)
    assert stub.calls == []


@pytest.mark.parametrize("case", ["out_short", "out_dtype", "out_noncontig", "container_short",
                                  "container_on_host", "out_on_host"])
def test_decode_rejects(stub, case):
    c, out = u8(512), t16(ROWS * COLS)
    if case == "out_short":
        out = t16(ROWS * COLS - 1)
    elif case == "out_dtype":
        out = f32(ROWS * COLS)
    elif case == "out_noncontig":
        out = t16(2, ROWS * COLS).t()
    elif case == "container_short":
        c = u8(500)
    elif case == "container_on_host":
        c = u8(512, device="cpu")
    elif case == "out_on_host":
        out = t16(ROWS * COLS, device="cpu")
    with pytest.raises((ValueError, TypeError)):
        wc.decode(H, c, out=out, stream=S)
    assert stub.calls == []


@pytest.mark.parametrize("case", ["container_short", "w_count", "work_short", "container_dtype"])
def test_encode_into_rejects(stub, case):
    n = ROWS * COLS
    w, c, work = t16(n), u8(512), u8(wc.workspace_bytes(n))
    if case == "container_short":
        c = u8(100)
    elif case == "w_count":
        w = t16(n - 1)
    elif case == "work_short":
        work = u8(wc.workspace_bytes(n) - 1)
    elif case == "container_dtype":
        c = t16(512)
    with pytest.raises((ValueError, TypeError)):
        wc.encode_into(H, w, c, work=work, stream=S)
    assert stub.calls == []


def test_build_dict_rejects_short_workspace(stub):
    with pytest.raises(ValueError):
        wc.build_dict(t16(1000), wc.BYTESPLIT, work=u8(wc.workspace_bytes(1000) - 16), stream=S)
    assert stub.calls == []
