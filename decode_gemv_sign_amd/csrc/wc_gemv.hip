// wc_gemv.hip — decode fused into GEMV, and the plain BF16 GEMV it is
// measured against.
//
// Page "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está listo
// para producción?", section "¿Qué significa “sin pérdida” para los pesos de
// un LLM?": the GPU keeps the coded weights, rebuilds the exact BF16 values in
// registers or shared memory and uses them at once in the matrix product.
// Page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%", section
// "Qué queda por demostrar": a dense prototype did this without the escape
// correction and was timed against a BF16 GEMV; here the escapes are applied
// inside the same kernel, tile by tile.
//
// y[b][r] = sum_c W[r][c] x[b][c].  One wave per row: per step each lane
// rebuilds 32 consecutive weights of the row (wc_tile.h), multiplies them with
// the matching x values by v_dot2_f32_bf16 (exact BF16 products, fp32
// accumulate), and at the row's end the 64 lane partials are summed by
// butterfly shuffles.  HBM-bound at batch 1 and 4: per weight bpw/8 bytes
// of container are read (x stays in L2).
//
// Rows whose length is not a multiple of 32 (a chunk would straddle two rows)
// take the generic kernels at the end of this file: one weight per lane per
// step, same definition, fp32 fused multiply-add.
#include "wc_launch.h"
#include "wc_tile.h"

namespace wc {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline float dot2(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, x), acc, false);
}

struct GemvArgs {
  const uint8_t* codes;
  const uint8_t* raw;
  const uint32_t* esc_pos;
  const uint8_t* esc_sym;
  const uint16_t* w;  // plain BF16 weights (comparator)
  const uint16_t* x;
  float* y;
  uint64_t rows, cols, n_esc, raw_padded;
  uint32_t batch;
  Dict dict;
};

// Multiply one lane chunk (16 weight pairs) with x[b][c0 .. c0+32) for every b.
template <int B>
__device__ inline void dot_chunk(const uint32_t w[16], const uint16_t* __restrict__ x,
                                 uint64_t cols, uint64_t c0, float acc[B]) {
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const u32x4* xp = (const u32x4*)(x + (uint64_t)b * cols + c0);
    float s0 = acc[b], s1 = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 xv = xp[k];
      s0 = dot2(w[4 * k + 0], xv[0], s0);
      s1 = dot2(w[4 * k + 1], xv[1], s1);
      s0 = dot2(w[4 * k + 2], xv[2], s0);
      s1 = dot2(w[4 * k + 3], xv[3], s1);
    }
    acc[b] = s0 + s1;
  }
}

template <int B>
__device__ inline void store_row(float acc[B], float* __restrict__ y, uint64_t rows, uint64_t r) {
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const float s = wave_sum_f32(acc[b]);
    if (lane_id() == 0) y[(uint64_t)b * rows + r] = s;
  }
}

template <int LAYOUT, int B>
__global__ __launch_bounds__(kBlockThreads) void k_decode_gemv(GemvArgs a) {
  __shared__ uint32_t T2[256];
  __shared__ uint32_t stage[kBlockThreads / kWave][kTile / 2];
  build_pair_table<LAYOUT>(T2, a.dict);
  __syncthreads();

  const int lane = lane_id();
  const int wib = (int)(threadIdx.x / kWave);
  const uint64_t r = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + (uint64_t)wib;
  if (r >= a.rows) return;

  const uint64_t cpr = a.cols / kChunk;  // chunks per row
  const uint64_t row_start = r * a.cols;
  uint64_t e = a.n_esc ? wave_lower_bound(a.esc_pos, a.n_esc, row_start) : 0;
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;

  for (uint64_t c0 = 0; c0 < cpr; c0 += kWave) {
    const uint64_t cc = c0 + (uint64_t)lane;
    const bool active = cc < cpr;
    Chunk c;
    if (active) {
      load_chunk_full<LAYOUT>(a.codes, a.raw, row_start / kChunk + cc, c);
    } else {
      c.codes = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 8; ++k) c.raw[k] = 0;
    }
    const uint32_t cnt = count_escapes(c.codes);
    uint32_t w[16];
    rebuild_chunk<LAYOUT>(T2, c, w);
    if (__ballot(cnt != 0)) {
      const uint32_t cnt_wave = wave_sum_u32(cnt);
      const uint64_t tile_start = row_start + c0 * kChunk;
      const uint64_t left = a.cols - c0 * kChunk;
      patch_tile<LAYOUT>(stage[wib], w, a.esc_pos, a.esc_sym, a.n_esc, e, cnt_wave, tile_start,
                         left >= kTile ? kTile : (uint32_t)left);
      e += cnt_wave;
    }
    if (active) dot_chunk<B>(w, a.x, a.cols, cc * kChunk, acc);
  }
  store_row<B>(acc, a.y, a.rows, r);
}

template <int B>
__global__ __launch_bounds__(kBlockThreads) void k_gemv_bf16(GemvArgs a) {
  const int lane = lane_id();
  const uint64_t r = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + threadIdx.x / kWave;
  if (r >= a.rows) return;
  const uint64_t cpr = a.cols / kChunk;
  const uint16_t* wr = a.w + r * a.cols;
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  for (uint64_t c0 = 0; c0 < cpr; c0 += kWave) {
    const uint64_t cc = c0 + (uint64_t)lane;
    if (cc < cpr) {
      const u32x4* wp = (const u32x4*)(wr + cc * kChunk);
      uint32_t w[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 v = __builtin_nontemporal_load(wp + k);
        w[4 * k] = v[0]; w[4 * k + 1] = v[1]; w[4 * k + 2] = v[2]; w[4 * k + 3] = v[3];
      }
      dot_chunk<B>(w, a.x, a.cols, cc * kChunk, acc);
    }
  }
  store_row<B>(acc, a.y, a.rows, r);
}

// ---- generic shapes (cols % 32 != 0): one weight per lane per step --------

__device__ inline float bf16f(uint32_t b) { return __uint_as_float(b << 16); }

template <int LAYOUT>
__global__ __launch_bounds__(kBlockThreads) void k_decode_gemv_generic(GemvArgs a) {
  __shared__ uint16_t dsym[16];
  if (threadIdx.x < 16) dsym[threadIdx.x] = a.dict.sym[threadIdx.x];
  __syncthreads();
  const int lane = lane_id();
  const uint64_t r = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + threadIdx.x / kWave;
  if (r >= a.rows) return;
  const uint64_t row_start = r * a.cols;
  const uint64_t n = a.rows * a.cols;
  const uint64_t raw_len = raw_bytes(LAYOUT, n);
  uint64_t e = a.n_esc ? wave_lower_bound(a.esc_pos, a.n_esc, row_start) : 0;
  float acc[WC_MAX_BATCH];
#pragma unroll
  for (int b = 0; b < (int)WC_MAX_BATCH; ++b) acc[b] = 0.0f;
  const uint64_t below = (1ull << lane) - 1ull;
  for (uint64_t c0 = 0; c0 < a.cols; c0 += kWave) {
    const uint64_t c = c0 + (uint64_t)lane;
    const bool valid = c < a.cols;
    const uint64_t i = row_start + c;
    const uint32_t code = valid ? (a.codes[i >> 1] >> (4u * (uint32_t)(i & 1u))) & 15u : 0u;
    const bool esc = valid && code == 15u;
    const uint64_t m = __ballot(esc);
    const uint64_t idx = e + (uint64_t)__popcll(m & below);
    uint32_t s = 0;
    if (esc) {
      if (idx < a.n_esc)
        s = LAYOUT == WC_LAYOUT_K15 ? (((const uint16_t*)a.esc_sym)[idx] & 0x1FFu) : a.esc_sym[idx];
    } else if (valid) {
      s = dsym[code];
    }
    uint32_t rawv = 0;
    if (valid) {
      if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
        rawv = a.raw[i];
      } else {
        const uint64_t bit = 7u * i, byte = bit >> 3;
        uint32_t v = a.raw[byte];
        if (byte + 1 < raw_len) v |= (uint32_t)a.raw[byte + 1] << 8;
        rawv = (v >> (uint32_t)(bit & 7u)) & 0x7Fu;
      }
    }
    const float wf = bf16f((s << (LAYOUT == WC_LAYOUT_K15 ? 7 : 8)) | rawv);
    if (valid) {
#pragma unroll
      for (int b = 0; b < (int)WC_MAX_BATCH; ++b)
        if (b < (int)a.batch) acc[b] = fmaf(wf, bf16f(a.x[(uint64_t)b * a.cols + c]), acc[b]);
    }
    e += (uint64_t)__popcll(m);
  }
#pragma unroll
  for (int b = 0; b < (int)WC_MAX_BATCH; ++b) {
    if (b < (int)a.batch) {
      const float s = wave_sum_f32(acc[b]);
      if (lane == 0) a.y[(uint64_t)b * a.rows + r] = s;
    }
  }
}

__global__ __launch_bounds__(kBlockThreads) void k_gemv_bf16_generic(GemvArgs a) {
  const int lane = lane_id();
  const uint64_t r = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + threadIdx.x / kWave;
  if (r >= a.rows) return;
  float acc[WC_MAX_BATCH];
#pragma unroll
  for (int b = 0; b < (int)WC_MAX_BATCH; ++b) acc[b] = 0.0f;
  for (uint64_t c = (uint64_t)lane; c < a.cols; c += kWave) {
    const float wf = bf16f(a.w[r * a.cols + c]);
#pragma unroll
    for (int b = 0; b < (int)WC_MAX_BATCH; ++b)
      if (b < (int)a.batch) acc[b] = fmaf(wf, bf16f(a.x[(uint64_t)b * a.cols + c]), acc[b]);
  }
#pragma unroll
  for (int b = 0; b < (int)WC_MAX_BATCH; ++b) {
    if (b < (int)a.batch) {
      const float s = wave_sum_f32(acc[b]);
      if (lane == 0) a.y[(uint64_t)b * a.rows + r] = s;
    }
  }
}

__global__ void k_fill_zero(float* y, uint64_t count) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) y[i] = 0.0f;
}

// ---- launchers -----------------------------------------------------------

static dim3 row_grid(uint64_t rows) {
  const uint64_t wpb = kBlockThreads / kWave;
  return dim3((unsigned)((rows + wpb - 1) / wpb));
}

template <int LAYOUT>
static void launch_fused_fast(const GemvArgs& a, hipStream_t s) {
  // Batch sizes 1, 2, 4, 8 and 16 have their own kernels; other sizes run as
  // a sum of those over consecutive slices of x and y.
  uint32_t done = 0;
  while (done < a.batch) {
    const uint32_t left = a.batch - done;
    GemvArgs p = a;
    p.x = a.x + (uint64_t)done * a.cols;
    p.y = a.y + (uint64_t)done * a.rows;
    uint32_t b = left >= 16 ? 16 : left >= 8 ? 8 : left >= 4 ? 4 : left >= 2 ? 2 : 1;
    p.batch = b;
    const dim3 g = row_grid(a.rows), t(kBlockThreads);
    switch (b) {
      case 16: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 16>), g, t, 0, s, p); break;
      case 8: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 8>), g, t, 0, s, p); break;
      case 4: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 4>), g, t, 0, s, p); break;
      case 2: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 2>), g, t, 0, s, p); break;
      default: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 1>), g, t, 0, s, p); break;
    }
    done += b;
  }
}

hipError_t launch_decode_gemv(const wc_header& h, const uint8_t* container, uint64_t rows,
                              uint64_t cols, const uint16_t* x, uint32_t batch, float* y,
                              hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols == 0) {
    const uint64_t count = rows * batch;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, y,
                       count);
    return hipGetLastError();
  }
  GemvArgs a;
  a.codes = container + h.off_codes;
  a.raw = container + h.off_raw;
  a.esc_pos = (const uint32_t*)(container + h.off_esc_pos);
  a.esc_sym = container + h.off_esc_sym;
  a.w = nullptr;
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.n_esc = h.n_esc;
  a.raw_padded = pad16(raw_bytes(h.layout, h.n));
  a.batch = batch;
  a.dict = dict_of(&h);
  if (cols % kChunk == 0) {
    if (h.layout == WC_LAYOUT_K15)
      launch_fused_fast<WC_LAYOUT_K15>(a, s);
    else
      launch_fused_fast<WC_LAYOUT_BYTESPLIT>(a, s);
  } else if (h.layout == WC_LAYOUT_K15) {
    hipLaunchKernelGGL(k_decode_gemv_generic<WC_LAYOUT_K15>, row_grid(rows), dim3(kBlockThreads), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL(k_decode_gemv_generic<WC_LAYOUT_BYTESPLIT>, row_grid(rows),
                       dim3(kBlockThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemv_bf16(const uint16_t* w, uint64_t rows, uint64_t cols, const uint16_t* x,
                            uint32_t batch, float* y, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (cols == 0) {
    const uint64_t count = rows * batch;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, y,
                       count);
    return hipGetLastError();
  }
  GemvArgs a = {};
  a.w = w;
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.batch = batch;
  if (cols % kChunk != 0) {
    hipLaunchKernelGGL(k_gemv_bf16_generic, row_grid(rows), dim3(kBlockThreads), 0, s, a);
    return hipGetLastError();
  }
  uint32_t done = 0;
  while (done < batch) {
    const uint32_t left = batch - done;
    GemvArgs p = a;
    p.x = x + (uint64_t)done * cols;
    p.y = y + (uint64_t)done * rows;
    uint32_t b = left >= 16 ? 16 : left >= 8 ? 8 : left >= 4 ? 4 : left >= 2 ? 2 : 1;
    p.batch = b;
    const dim3 g = row_grid(rows), t(kBlockThreads);
    switch (b) {
      case 16: hipLaunchKernelGGL(k_gemv_bf16<16>, g, t, 0, s, p); break;
      case 8: hipLaunchKernelGGL(k_gemv_bf16<8>, g, t, 0, s, p); break;
      case 4: hipLaunchKernelGGL(k_gemv_bf16<4>, g, t, 0, s, p); break;
      case 2: hipLaunchKernelGGL(k_gemv_bf16<2>, g, t, 0, s, p); break;
      default: hipLaunchKernelGGL(k_gemv_bf16<1>, g, t, 0, s, p); break;
    }
    done += b;
  }
  return hipGetLastError();
}

}  // namespace wc
