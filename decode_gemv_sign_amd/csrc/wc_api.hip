// wc_api.hip — the C ABI of libwc (declared and documented in include/wc.h).
//
// Argument checks happen here, before anything is enqueued; kernels and
// launch geometry live in wc_encode.hip, wc_decode.hip and wc_gemv.hip.
// The library allocates no device or host memory: every buffer is the
// caller's (wc_encode_noalloc's fixed scratch array is part of the loaded
// code object, see wc_encode.hip).
#include <string.h>

#include "wc_launch.h"

static_assert(sizeof(wc_header) == WC_HEADER_BYTES, "wc_header must be exactly 128 bytes");
static_assert(sizeof(wc::DictResult) == 48, "DictResult layout");

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? WC_OK : WC_E_HIP; }

bool layout_ok(int layout) {
  return layout == WC_LAYOUT_BYTESPLIT || layout == WC_LAYOUT_K15 || layout == WC_LAYOUT_RAW ||
         layout == WC_LAYOUT_AUTO;
}

}  // namespace

extern "C" int wc_build_dict(int layout, const uint16_t* d_w, uint64_t n, void* d_work,
                             size_t work_bytes, void* stream, wc_header* h_out) {
  // WC_COMPACT asks for the compact escape form of a coded layout
  const bool compact = (layout & WC_COMPACT) != 0;
  layout &= ~WC_COMPACT;
  if (!h_out || !layout_ok(layout)) return WC_E_ARG;
  const uint32_t cflags = compact ? WC_FLAG_COMPACT : 0u;
  if (n >= (1ull << 32)) return WC_E_SIZE;
  if (n && (!d_w || !wc::aligned16(d_w))) return WC_E_ARG;
  if (!d_work || !wc::aligned16(d_work)) return WC_E_ARG;
  if (work_bytes < WC_WORKSPACE_BYTES(n)) return WC_E_SIZE;
  hipStream_t s = (hipStream_t)stream;

  // r[0]: the dictionary of `layout` (byte-split's under AUTO), r[1]: K15's
  // under AUTO; the raw layout has none
  wc::DictResult r[2];
  memset(r, 0, sizeof r);
  if (n && layout != WC_LAYOUT_RAW) {
    hipError_t e = wc::launch_build_dict(layout, d_w, n, (uint8_t*)d_work, s);
    if (e != hipSuccess) return WC_E_HIP;
    static_assert(wc::kWorkResult2 == wc::kWorkResult + sizeof(wc::DictResult), "results adjacent");
    const size_t nres = layout == WC_LAYOUT_AUTO ? 2 : 1;
    e = hipMemcpyAsync(r, (uint8_t*)d_work + wc::kWorkResult, nres * sizeof(wc::DictResult),
                       hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return WC_E_HIP;
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return WC_E_HIP;
    for (int k = 0; k < (layout == WC_LAYOUT_AUTO ? 2 : 1); ++k)
      if (r[k].n_dict > 15 || r[k].n_esc > n) return WC_E_HIP;  // not a valid result: the device work failed
  }
  if (layout == WC_LAYOUT_AUTO) {
    // the smallest container, ties to the lower layout number
    const uint64_t t0 = wc::geometry(WC_LAYOUT_BYTESPLIT, n, r[0].n_esc, cflags).total;
    const uint64_t t1 = wc::geometry(WC_LAYOUT_K15, n, r[1].n_esc, cflags).total;
    const uint64_t t2 = wc::geometry(WC_LAYOUT_RAW, n, 0).total;
    layout = WC_LAYOUT_BYTESPLIT;
    uint64_t best = t0;
    if (t1 < best) {
      layout = WC_LAYOUT_K15;
      best = t1;
      r[0] = r[1];
    }
    if (t2 < best) layout = WC_LAYOUT_RAW;
  }
  const wc::DictResult& rr = r[0];
  wc_header h;
  memset(&h, 0, sizeof h);
  h.magic = WC_MAGIC;
  h.version = WC_VERSION;
  h.layout = (uint8_t)layout;
  h.n = n;
  if (layout != WC_LAYOUT_RAW) {
    h.n_dict = (uint8_t)rr.n_dict;
    h.n_esc = rr.n_esc;
    for (int k = 0; k < 16; ++k) h.dict[k] = k < (int)rr.n_dict ? rr.dict[k] : 0;
    h.flags = (uint8_t)cflags;
  }
  const wc::Geometry g = wc::geometry(layout, n, h.n_esc, h.flags);
  h.off_codes = g.off_codes;
  h.off_raw = g.off_raw;
  h.off_esc_pos = g.off_esc_pos;
  h.off_esc_sym = g.off_esc_sym;
  h.off_esc_idx = g.off_esc_idx;
  h.total_bytes = g.total;
  *h_out = h;
  return WC_OK;
}

extern "C" int wc_encode(const wc_header* h, const uint16_t* d_w, uint8_t* d_container,
                         size_t container_bytes, void* d_work, size_t work_bytes, void* stream) {
  if (!h || !d_container || !wc::aligned16(d_container)) return WC_E_ARG;
  const int v = wc::validate_header(h);
  if (v != WC_OK) return v;
  if (h->n && (!d_w || !wc::aligned16(d_w))) return WC_E_ARG;
  if (!d_work || !wc::aligned16(d_work)) return WC_E_ARG;
  if (work_bytes < WC_WORKSPACE_BYTES(h->n) || container_bytes < h->total_bytes) return WC_E_SIZE;
  return hip_status(wc::launch_encode(*h, d_w, d_container, (uint8_t*)d_work, (hipStream_t)stream));
}

extern "C" int wc_encode_noalloc(const wc_header* h, const uint16_t* d_w, uint8_t* d_container,
                                 size_t container_bytes, void* stream) {
  if (!h || !d_container || !wc::aligned16(d_container)) return WC_E_ARG;
  const int v = wc::validate_header(h);
  if (v != WC_OK) return v;
  if (h->n > WC_NOALLOC_MAX_N) return WC_E_SIZE;
  if (h->n && (!d_w || !wc::aligned16(d_w))) return WC_E_ARG;
  if (container_bytes < h->total_bytes) return WC_E_SIZE;
  return hip_status(wc::launch_encode_noalloc(*h, d_w, d_container, (hipStream_t)stream));
}

extern "C" int wc_decode(const wc_header* h, const uint8_t* d_container, size_t container_bytes,
                         uint16_t* d_out, void* stream) {
  if (!h || !d_container || !wc::aligned16(d_container)) return WC_E_ARG;
  const int v = wc::validate_header(h);
  if (v != WC_OK) return v;
  if (container_bytes < h->total_bytes) return WC_E_SIZE;
  if (h->n && (!d_out || !wc::aligned16(d_out))) return WC_E_ARG;
  return hip_status(wc::launch_decode(*h, d_container, d_out, (hipStream_t)stream));
}

extern "C" int wc_decode_gemv(const wc_header* h, const uint8_t* d_container,
                              size_t container_bytes, uint64_t rows, uint64_t cols,
                              const uint16_t* d_x, uint32_t batch, float* d_y, void* stream) {
  if (!h || !d_container || !wc::aligned16(d_container)) return WC_E_ARG;
  const int v = wc::validate_header(h);
  if (v != WC_OK) return v;
  if (container_bytes < h->total_bytes) return WC_E_SIZE;
  if (batch < 1 || batch > WC_MAX_BATCH) return WC_E_UNSUPPORTED;
  if (cols && rows > h->n / cols) return WC_E_ARG;
  if (rows * cols != h->n) return WC_E_ARG;
  if (rows && (!d_y || ((uintptr_t)d_y & 3u))) return WC_E_ARG;
  if (rows && cols && (!d_x || !wc::aligned16(d_x))) return WC_E_ARG;
  return hip_status(
      wc::launch_decode_gemv(*h, d_container, rows, cols, d_x, batch, d_y, (hipStream_t)stream));
}

extern "C" int wc_gemv_bf16(const uint16_t* d_w, uint64_t rows, uint64_t cols, const uint16_t* d_x,
                            uint32_t batch, float* d_y, void* stream) {
  if (batch < 1 || batch > WC_MAX_BATCH) return WC_E_UNSUPPORTED;
  if (cols && rows >= (1ull << 62) / cols) return WC_E_SIZE;
  if (rows && (!d_y || ((uintptr_t)d_y & 3u))) return WC_E_ARG;
  if (rows && cols && (!d_w || !d_x || !wc::aligned16(d_w) || !wc::aligned16(d_x))) return WC_E_ARG;
  return hip_status(wc::launch_gemv_bf16(d_w, rows, cols, d_x, batch, d_y, (hipStream_t)stream));
}

extern "C" int wc_bits_per_weight(const wc_header* h, double* bpw, double* payload_bpw) {
  if (!h || !bpw || !payload_bpw) return WC_E_ARG;
  const int v = wc::validate_header(h);
  if (v != WC_OK) return v;
  if (h->n == 0) return WC_E_ARG;
  const uint64_t payload = wc::code_bytes(h->layout, h->n) + wc::raw_bytes(h->layout, h->n) +
                           wc::pos_bytes(h->flags, h->n_esc) + wc::sym_bytes(h->layout) * h->n_esc +
                           4u * wc::index_entries(h->n, h->n_esc);
  *bpw = 8.0 * (double)h->total_bytes / (double)h->n;
  *payload_bpw = 8.0 * (double)payload / (double)h->n;
  return WC_OK;
}
