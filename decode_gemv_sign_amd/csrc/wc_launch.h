// wc_launch.h — internal launchers of libwc's kernels (host side).  Each
// returns a hipError_t from the launch; argument checks happen in wc_api.hip.
#pragma once

#include "wc_common.h"

namespace wc {

// Byte offsets inside the caller's workspace (WC_WORKSPACE_BYTES(n) bytes).
constexpr int kHistGlobal = 8;          // copies of the global histogram (blocks spread over them)
constexpr size_t kWorkHist = 0;         // u32[kHistGlobal][512] symbol counts
constexpr size_t kWorkResult = 16384;   // DictResult (of the layout asked for; byte-split's under AUTO)
constexpr size_t kWorkResult2 = 16432;  // DictResult of K15 under AUTO
constexpr size_t kWorkBlocks = 20480;   // encode: u32[nblk] escape counts, u32[nblk] offsets, then
                                        // the symbol stage (WC_STAGE_SYMBOLS u16 per block)
static_assert(kWorkHist + 4u * 512u * kHistGlobal <= kWorkResult, "histogram copies fit");

struct DictResult {
  uint32_t n_dict;
  uint32_t reserved;
  uint64_t n_esc;
  uint16_t dict[16];
};

// Compute units of the current device (cached per device).
inline uint32_t cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return (uint32_t)cached[dev];
}

// layout WC_LAYOUT_AUTO ranks both symbol kinds (results at kWorkResult and
// kWorkResult2).
hipError_t launch_build_dict(int layout, const uint16_t* w, uint64_t n, uint8_t* work,
                             hipStream_t s);
// Raw layout (wc_decode.hip): the weights copied into / out of the container.
hipError_t launch_encode_raw(const wc_header& h, const uint16_t* w, uint8_t* container,
                             hipStream_t s);
hipError_t launch_decode_raw(const wc_header& h, const uint8_t* container, uint16_t* out,
                             hipStream_t s);
hipError_t launch_encode(const wc_header& h, const uint16_t* w, uint8_t* container, uint8_t* work,
                         hipStream_t s);
// The same with the library's own per-GPU scratch (no workspace argument);
// h.n <= WC_NOALLOC_MAX_N.
hipError_t launch_encode_noalloc(const wc_header& h, const uint16_t* w, uint8_t* container,
                                 hipStream_t s);
hipError_t launch_decode(const wc_header& h, const uint8_t* container, uint16_t* out,
                         hipStream_t s);
hipError_t launch_decode_gemv(const wc_header& h, const uint8_t* container, uint64_t rows,
                              uint64_t cols, const uint16_t* x, uint32_t batch, float* y,
                              hipStream_t s);
// Matrix-core paths (wc_gemm.hip): cols a multiple of 32, batch 1..16.
bool gemm_mfma_fits(uint64_t rows, uint64_t cols, uint32_t batch);
// Wide batches on the matrix cores (from 17 on tensors of 2^26 weights or
// more, else from 33, up to WC_MAX_BATCH): cols a multiple of 128.
bool gemm_wide_fits(uint64_t rows, uint64_t cols, uint32_t batch);
// y[0 .. count) = 0 (wc_gemv.hip; a kernel rather than a memset, so that a
// captured launch sequence holds no memset node).
__global__ void k_fill_zero(float* y, uint64_t count);
hipError_t launch_decode_gemm_mfma(const wc_header& h, const uint8_t* container, uint64_t rows,
                                   uint64_t cols, const uint16_t* x, uint32_t batch, float* y,
                                   hipStream_t s);
hipError_t launch_gemm_bf16_mfma(const uint16_t* w, uint64_t rows, uint64_t cols,
                                 const uint16_t* x, uint32_t batch, float* y, hipStream_t s);
hipError_t launch_gemv_bf16(const uint16_t* w, uint64_t rows, uint64_t cols, const uint16_t* x,
                            uint32_t batch, float* y, hipStream_t s);

}  // namespace wc
