"""decode_gemv_sign_amd — Python binding of libwc (include/wc.h).

Lossless BF16 sign+exponent coding on AMD MI355X: a per-tensor 15-entry
dictionary of sign+exponent symbols, 4-bit codes, an exact escape stream,
and the raw part kept as stored (byte-split: the low byte; K15: the 7-bit
mantissa) — page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%",
section "Cómo funciona la compresión" — with exact decode and decode fused
into GEMV (page "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está
listo para producción?", section "¿Qué significa “sin pérdida” para los pesos
de un LLM?").

This module only marshals arguments: every step runs in the HIP kernels of
libwc.so, on the caller's current torch stream.  PyTorch provides device
memory and streams.  There is no CPU fallback: importing this package
without a built libwc.so raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first, so libwc binds to the HIP runtime torch already uses

__all__ = [
    "BYTESPLIT", "K15", "RAW", "AUTO", "COMPACT", "FLAG_COMPACT", "Header", "WCError", "workspace_bytes", "build_dict", "encode_into", "encode_into_noalloc",
    "encode", "decode", "decode_gemv", "gemv_bf16", "bits_per_weight", "read_header",
    "crc32", "container_crcs", "artifact_write", "artifact_entries", "artifact_read",
    "artifact_verify", "LIB_PATH",
]

BYTESPLIT = 0
K15 = 1
RAW = 2   # fallback layout: the BF16 bit patterns as stored
AUTO = 3  # build_dict / encode only: the smallest of the three
COMPACT = 0x10  # OR into a layout: escape symbols only (header flag FLAG_COMPACT)
FLAG_COMPACT = 1
MAX_BATCH = 256
STAGE_SYMBOLS = 256  # WC_STAGE_SYMBOLS
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwc.so")

_CODES = {0: "WC_OK", -1: "WC_E_ARG", -2: "WC_E_SIZE", -3: "WC_E_CORRUPT", -4: "WC_E_HIP",
          -5: "WC_E_UNSUPPORTED", -6: "WC_E_IO"}


class WCError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_CODES.get(code, code)}")
        self.code = code


class Header(ctypes.Structure):
    """wc_header: the first 128 bytes of every container."""
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint16), ("layout", ctypes.c_uint8),
        ("n_dict", ctypes.c_uint8), ("n", ctypes.c_uint64), ("n_esc", ctypes.c_uint64),
        ("dict", ctypes.c_uint16 * 16), ("off_codes", ctypes.c_uint64),
        ("off_raw", ctypes.c_uint64), ("off_esc_pos", ctypes.c_uint64),
        ("off_esc_sym", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
        ("off_esc_idx", ctypes.c_uint64), ("flags", ctypes.c_uint8),
        ("reserved", ctypes.c_uint8 * 23),
    ]

    def to_bytes(self) -> bytes:
        return ctypes.string_at(ctypes.addressof(self), ctypes.sizeof(self))

    @classmethod
    def from_bytes(cls, b: bytes) -> "Header":
        if len(b) < 128:
            raise ValueError("a header is 128 bytes")
        return cls.from_buffer_copy(bytes(b[:128]))


assert ctypes.sizeof(Header) == 128


class ArtifactInfo(ctypes.Structure):
    """wc_artifact_info: one entry of a serialized artifact."""
    _fields_ = [
        ("name", ctypes.c_char * 96), ("ndim", ctypes.c_uint32), ("layout", ctypes.c_uint32),
        ("shape", ctypes.c_uint64 * 4), ("offset", ctypes.c_uint64), ("bytes", ctypes.c_uint64),
        ("src_crc", ctypes.c_uint32), ("stream_crc", ctypes.c_uint32 * 6),
        ("reserved", ctypes.c_uint32),
    ]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m decode_gemv_sign_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    U64 = ctypes.c_uint64
    HP = ctypes.POINTER(Header)
    lib.wc_build_dict.argtypes = [ctypes.c_int, P, U64, P, ctypes.c_size_t, P, HP]
    lib.wc_encode.argtypes = [HP, P, P, ctypes.c_size_t, P, ctypes.c_size_t, P]
    lib.wc_encode_noalloc.argtypes = [HP, P, P, ctypes.c_size_t, P]
    lib.wc_decode.argtypes = [HP, P, ctypes.c_size_t, P, P]
    lib.wc_decode_gemv.argtypes = [HP, P, ctypes.c_size_t, U64, U64, P, ctypes.c_uint32, P, P]
    lib.wc_gemv_bf16.argtypes = [P, U64, U64, P, ctypes.c_uint32, P, P]
    lib.wc_bits_per_weight.argtypes = [HP, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)]
    lib.wc_crc32.argtypes = [ctypes.c_uint32, P, ctypes.c_size_t]
    lib.wc_crc32.restype = ctypes.c_uint32
    lib.wc_container_crcs.argtypes = [P, ctypes.c_size_t, P]
    lib.wc_artifact_write.argtypes = [ctypes.c_char_p, ctypes.c_uint32,
                                      ctypes.POINTER(ctypes.c_char_p), P, P,
                                      ctypes.POINTER(ctypes.c_void_p), P, P]
    lib.wc_artifact_count.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_uint32)]
    lib.wc_artifact_entry.argtypes = [ctypes.c_char_p, ctypes.c_uint32,
                                      ctypes.POINTER(ArtifactInfo)]
    lib.wc_artifact_read.argtypes = [ctypes.c_char_p, ctypes.c_uint32, P, ctypes.c_size_t]
    for f in (lib.wc_build_dict, lib.wc_encode, lib.wc_encode_noalloc, lib.wc_decode, lib.wc_decode_gemv,
              lib.wc_gemv_bf16, lib.wc_bits_per_weight, lib.wc_container_crcs,
              lib.wc_artifact_write, lib.wc_artifact_count, lib.wc_artifact_entry,
              lib.wc_artifact_read):
        f.restype = ctypes.c_int
    return lib


_lib = _load()


def use_library(path: str):
    """Bind this module to another build of libwc (e.g. a tuning variant)."""
    global _lib
    _lib = _load(path)


def _check(st: int, what: str):
    if st != 0:
        raise WCError(st, what)


def _stream(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_device(t: torch.Tensor) -> bool:
    """True for a tensor in GPU memory (the library takes device pointers only)."""
    return t.device.type == "cuda"


def _bits16(t: torch.Tensor, what: str) -> torch.Tensor:
    """A contiguous 16-bit device tensor viewed as raw BF16 bit patterns."""
    if not _on_device(t):
        raise ValueError(f"{what} must be a device tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{what} must hold BF16 bit patterns (bfloat16, int16 or uint16)")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _bytes(t: torch.Tensor, what: str, need: int) -> torch.Tensor:
    """A contiguous uint8 device tensor of at least `need` bytes."""
    if not _on_device(t):
        raise ValueError(f"{what} must be a device tensor")
    if t.dtype != torch.uint8:
        raise TypeError(f"{what} must be a uint8 tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() < need:
        raise ValueError(f"{what} holds {t.numel()} bytes, {need} needed")
    return t


def _same_device(what: str, *ts: torch.Tensor):
    devs = {t.device for t in ts}
    if len(devs) > 1:
        raise ValueError(f"{what}: tensors on different devices {sorted(map(str, devs))}")


def _batch_of(x: torch.Tensor, cols: int, what: str = "x") -> int:
    """Rows of x, which must be exactly [batch, cols] (or [cols] for batch 1):
    the library reads batch * cols values and cannot check that itself."""
    if x.dim() == 1:
        batch = 1
    elif x.dim() == 2:
        batch = x.shape[0]
    else:
        raise ValueError(f"{what} must be [batch, cols] or [cols], got {tuple(x.shape)}")
    if x.shape[-1] != cols or x.numel() != batch * cols:
        raise ValueError(f"{what} has shape {tuple(x.shape)}, expected ({batch}, {cols})")
    if not 1 <= batch <= MAX_BATCH:
        raise ValueError(f"batch {batch} outside 1..{MAX_BATCH}")
    return batch


def _gemv_out(out: torch.Tensor, batch: int, rows: int, what: str = "out") -> torch.Tensor:
    """y must be fp32 [batch, rows] (or [rows] for batch 1), contiguous, on the device."""
    if not _on_device(out):
        raise ValueError(f"{what} must be a device tensor")
    if out.dtype != torch.float32:
        raise TypeError(f"{what} must be float32")
    if not out.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    ok = tuple(out.shape) == (batch, rows) or (batch == 1 and tuple(out.shape) == (rows,))
    if not ok:
        raise ValueError(f"{what} has shape {tuple(out.shape)}, expected ({batch}, {rows})")
    return out


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() else 0)


def workspace_bytes(n: int) -> int:
    """WC_WORKSPACE_BYTES(n)."""
    return 20528 + (16 + 6 * STAGE_SYMBOLS) * ((n + 8191) // 8192)


def _workspace(n: int, device) -> torch.Tensor:
    return torch.empty(workspace_bytes(n), dtype=torch.uint8, device=device)


def build_dict(w: torch.Tensor, layout: int, work: torch.Tensor | None = None,
               stream=None) -> Header:
    """wc_build_dict: dictionary + complete container header for w (waits)."""
    w = _bits16(w, "w")
    n = w.numel()
    if work is None:
        work = _workspace(n, w.device)
    _bytes(work, "work", workspace_bytes(n))
    _same_device("build_dict", w, work)
    h = Header()
    _check(_lib.wc_build_dict(layout, _ptr(w), n, _ptr(work), work.numel(), _stream(stream),
                              ctypes.byref(h)), "wc_build_dict")
    return h


def encode_into(h: Header, w: torch.Tensor, container: torch.Tensor,
                work: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """wc_encode into a caller-allocated uint8 container (asynchronous)."""
    w = _bits16(w, "w")
    if w.numel() != h.n:
        raise ValueError(f"w has {w.numel()} weights, the header {h.n}")
    _bytes(container, "container", h.total_bytes)
    if work is None:
        work = _workspace(w.numel(), w.device)
    _bytes(work, "work", workspace_bytes(w.numel()))
    _same_device("encode_into", w, container, work)
    _check(_lib.wc_encode(ctypes.byref(h), _ptr(w), _ptr(container), container.numel(),
                          _ptr(work), work.numel(), _stream(stream)), "wc_encode")
    return container


def encode_into_noalloc(h: Header, w: torch.Tensor, container: torch.Tensor,
                        stream=None) -> torch.Tensor:
    """wc_encode_noalloc: as encode_into, with the library's own per-GPU
    scratch instead of a workspace (nothing is allocated; calls that overlap
    on one GPU race)."""
    w = _bits16(w, "w")
    if w.numel() != h.n:
        raise ValueError(f"w has {w.numel()} weights, the header {h.n}")
    _bytes(container, "container", h.total_bytes)
    _same_device("encode_into_noalloc", w, container)
    _check(_lib.wc_encode_noalloc(ctypes.byref(h), _ptr(w), _ptr(container), container.numel(),
                                  _stream(stream)), "wc_encode_noalloc")
    return container


def encode(w: torch.Tensor, layout: int, stream=None):
    """(header, container): dictionary, then the whole container on the device."""
    w = _bits16(w, "w")
    work = _workspace(w.numel(), w.device)
    h = build_dict(w, layout, work, stream)
    c = torch.empty(h.total_bytes, dtype=torch.uint8, device=w.device)
    encode_into(h, w, c, work, stream)
    return h, c


def read_header(container: torch.Tensor) -> Header:
    """Copy a container's first 128 bytes back to the host (synchronises)."""
    return Header.from_bytes(container[:128].cpu().numpy().tobytes())


def decode(h: Header, container: torch.Tensor, out: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """wc_decode: the n BF16 bit patterns (int16 tensor unless `out` is given)."""
    _bytes(container, "container", h.total_bytes)
    if out is None:
        out = torch.empty(h.n, dtype=torch.int16, device=container.device)
    out = _bits16(out, "out")
    if out.numel() < h.n:
        raise ValueError(f"out holds {out.numel()} weights, {h.n} needed")
    _same_device("decode", container, out)
    _check(_lib.wc_decode(ctypes.byref(h), _ptr(container), container.numel(), _ptr(out),
                          _stream(stream)), "wc_decode")
    return out


def decode_gemv(h: Header, container: torch.Tensor, rows: int, cols: int, x: torch.Tensor,
                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """wc_decode_gemv: y [batch, rows] fp32 for x [batch, cols] BF16."""
    _bytes(container, "container", h.total_bytes)
    if rows * cols != h.n:
        raise ValueError(f"rows * cols = {rows * cols}, the header holds {h.n} weights")
    x = _bits16(x, "x")
    batch = _batch_of(x, cols)
    if out is None:
        out = torch.empty((batch, rows), dtype=torch.float32, device=container.device)
    _gemv_out(out, batch, rows)
    _same_device("decode_gemv", container, x, out)
    _check(_lib.wc_decode_gemv(ctypes.byref(h), _ptr(container), container.numel(), rows, cols,
                               _ptr(x), batch, _ptr(out), _stream(stream)), "wc_decode_gemv")
    return out


def gemv_bf16(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """wc_gemv_bf16: plain BF16 GEMV, W [rows, cols], x [batch, cols] -> [batch, rows]."""
    w = _bits16(w, "w")
    if w.dim() != 2:
        raise ValueError(f"w must be [rows, cols], got {tuple(w.shape)}")
    x = _bits16(x, "x")
    rows, cols = w.shape
    batch = _batch_of(x, cols)
    if out is None:
        out = torch.empty((batch, rows), dtype=torch.float32, device=w.device)
    _gemv_out(out, batch, rows)
    _same_device("gemv_bf16", w, x, out)
    _check(_lib.wc_gemv_bf16(_ptr(w), rows, cols, _ptr(x), batch, _ptr(out), _stream(stream)),
           "wc_gemv_bf16")
    return out


def bits_per_weight(h: Header):
    """(bits/weight with all overhead, payload bits/weight)."""
    b = ctypes.c_double()
    p = ctypes.c_double()
    _check(_lib.wc_bits_per_weight(ctypes.byref(h), ctypes.byref(b), ctypes.byref(p)),
           "wc_bits_per_weight")
    return b.value, p.value


# ---- serialized artifact (host side; include/wc.h) --------------------------

def _host_u8(a):
    import numpy as np
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a).view(np.uint8).reshape(-1)


def crc32(data, crc: int = 0) -> int:
    """wc_crc32 over a host buffer (numpy array, bytes or CPU/device tensor)."""
    if isinstance(data, (bytes, bytearray)):
        buf = ctypes.create_string_buffer(bytes(data), len(data))
        return _lib.wc_crc32(crc, buf, len(data))
    a = _host_u8(data)
    return _lib.wc_crc32(crc, ctypes.c_void_p(a.ctypes.data), a.size)


def container_crcs(container):
    """The six region CRCs of a container (host copy)."""
    a = _host_u8(container)
    out = (ctypes.c_uint32 * 6)()
    _check(_lib.wc_container_crcs(ctypes.c_void_p(a.ctypes.data), a.size, out), "wc_container_crcs")
    return list(out)


def artifact_write(path: str, items):
    """items: (name, shape, container, src_crc) per tensor; containers are
    copied to the host if they are device tensors."""
    import numpy as np
    items = list(items)
    n = len(items)
    names = (ctypes.c_char_p * max(n, 1))(*[it[0].encode() for it in items])
    ndims = np.zeros(max(n, 1), dtype=np.uint32)
    shapes = np.zeros((max(n, 1), 4), dtype=np.uint64)
    hosts = [_host_u8(it[2]) for it in items]
    ptrs = (ctypes.c_void_p * max(n, 1))(*[h.ctypes.data for h in hosts])
    sizes = np.array([h.size for h in hosts] or [0], dtype=np.uint64)
    crcs = np.array([it[3] for it in items] or [0], dtype=np.uint32)
    for i, it in enumerate(items):
        shp = tuple(int(d) for d in it[1])
        ndims[i] = len(shp)
        shapes[i, :len(shp)] = shp
    _check(_lib.wc_artifact_write(path.encode(), n, names, ctypes.c_void_p(ndims.ctypes.data),
                                  ctypes.c_void_p(shapes.ctypes.data), ptrs,
                                  ctypes.c_void_p(sizes.ctypes.data),
                                  ctypes.c_void_p(crcs.ctypes.data)), "wc_artifact_write")


def artifact_entries(path: str):
    """Every entry's metadata (file header and every entry checked)."""
    cnt = ctypes.c_uint32()
    _check(_lib.wc_artifact_count(path.encode(), ctypes.byref(cnt)), "wc_artifact_count")
    out = []
    for i in range(cnt.value):
        info = ArtifactInfo()
        _check(_lib.wc_artifact_entry(path.encode(), i, ctypes.byref(info)), "wc_artifact_entry")
        out.append({"name": info.name.decode(), "shape": tuple(info.shape[:info.ndim]),
                    "layout": info.layout, "offset": info.offset, "bytes": info.bytes,
                    "src_crc": info.src_crc, "stream_crc": list(info.stream_crc)})
    return out


def artifact_read(path: str, i: int):
    """Container i as a host uint8 array, after every CRC check."""
    import numpy as np
    info = ArtifactInfo()
    _check(_lib.wc_artifact_entry(path.encode(), i, ctypes.byref(info)), "wc_artifact_entry")
    buf = np.empty(info.bytes, dtype=np.uint8)
    _check(_lib.wc_artifact_read(path.encode(), i, ctypes.c_void_p(buf.ctypes.data), buf.size),
           "wc_artifact_read")
    return buf


def artifact_verify(path: str, device="cuda:0"):
    """Streams every tensor of the artifact through the GPU: read (CRCs
    checked), upload, exact decode, and the decoded values' CRC-32 against
    the source's.  Returns (name, matches, bits/weight) per tensor."""
    out = []
    for i, e in enumerate(artifact_entries(path)):
        host = artifact_read(path, i)
        c = torch.from_numpy(host).to(device)
        h = Header.from_bytes(host[:128].tobytes())
        dec = decode(h, c)
        got = crc32(dec)
        bpw = bits_per_weight(h)[0] if h.n else 0.0
        out.append((e["name"], got == e["src_crc"], bpw))
    return out
