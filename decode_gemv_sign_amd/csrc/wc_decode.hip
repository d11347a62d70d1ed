// wc_decode.hip — exact decode of a container into BF16 bit patterns.
//
// Page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%", section
// "Cómo funciona la compresión": the high byte (byte-split) or the 9-bit
// sign+exponent symbol (K15) is rebuilt from the dictionary, the code
// indices and the exact escape stream; the stored raw part is unchanged.
//
// HBM-bound: per weight it reads bpw/8 bytes of container and writes 2 bytes.
// Each wave owns a contiguous run of 2048-weight tiles, so the escape cursor
// is found once per wave (one 64-ary search of the position stream) and then
// advanced by each tile's code-15 count.  Tiles without escapes (a wave-wide
// ballot) store straight from registers with 16-byte non-temporal stores;
// tiles with escapes are patched in LDS first (wc_tile.h).
#include "wc_launch.h"
#include "wc_tile.h"

namespace wc {

struct DecodeArgs {
  const uint8_t* codes;
  const uint8_t* raw;
  const uint32_t* esc_pos;
  const uint8_t* esc_sym;
  uint16_t* out;
  uint64_t n, n_esc, raw_padded, n_tiles, tiles_per_wave;
  Dict dict;
};

template <int LAYOUT>
__global__ __launch_bounds__(kBlockThreads) void k_decode(DecodeArgs a) {
  __shared__ uint32_t T2[256];
  __shared__ uint32_t stage[kBlockThreads / kWave][kTile / 2];
  build_pair_table<LAYOUT>(T2, a.dict);
  __syncthreads();

  const int lane = lane_id();
  const int wib = (int)(threadIdx.x / kWave);
  const uint64_t wave = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + (uint64_t)wib;
  const uint64_t t0 = wave * a.tiles_per_wave;
  const uint64_t t1 = t0 + a.tiles_per_wave < a.n_tiles ? t0 + a.tiles_per_wave : a.n_tiles;
  if (t0 >= t1) return;

  uint64_t e = a.n_esc ? wave_lower_bound(a.esc_pos, a.n_esc, t0 * kTile) : 0;
  for (uint64_t t = t0; t < t1; ++t) {
    const uint64_t chunk = t * kWave + (uint64_t)lane;
    const uint64_t base = chunk * kChunk;
    const uint32_t valid = base < a.n ? (a.n - base >= kChunk ? kChunk : (uint32_t)(a.n - base)) : 0;
    Chunk c;
    if (valid == kChunk) {
      load_chunk_full<LAYOUT>(a.codes, a.raw, chunk, c);
    } else if (valid) {
      load_chunk_partial<LAYOUT>(a.codes, a.raw, chunk, valid, a.raw_padded, c);
    } else {
      c.codes = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 8; ++k) c.raw[k] = 0;
    }
    const uint32_t cnt = count_escapes(c.codes);
    uint32_t out[16];
    rebuild_chunk<LAYOUT>(T2, c, out);
    if (__ballot(cnt != 0)) {
      const uint32_t cnt_wave = wave_sum_u32(cnt);
      const uint64_t tile_start = t * kTile;
      const uint32_t tile_len = a.n - tile_start >= kTile ? kTile : (uint32_t)(a.n - tile_start);
      patch_tile<LAYOUT>(stage[wib], out, a.esc_pos, a.esc_sym, a.n_esc, e, cnt_wave, tile_start,
                         tile_len);
      e += cnt_wave;
    }
    if (valid == kChunk) {
      u32x4* dst = (u32x4*)(a.out + base);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        __builtin_nontemporal_store(u32x4{out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]},
                                    dst + k);
    } else if (valid) {
      for (uint32_t i = 0; i < valid; ++i)
        a.out[base + i] = (uint16_t)(out[i >> 1] >> (16u * (i & 1u)));
    }
  }
}

hipError_t launch_decode(const wc_header& h, const uint8_t* container, uint16_t* out,
                         hipStream_t s) {
  if (h.n == 0) return hipSuccess;
  DecodeArgs a;
  a.codes = container + h.off_codes;
  a.raw = container + h.off_raw;
  a.esc_pos = (const uint32_t*)(container + h.off_esc_pos);
  a.esc_sym = container + h.off_esc_sym;
  a.out = out;
  a.n = h.n;
  a.n_esc = h.n_esc;
  a.raw_padded = pad16(raw_bytes(h.layout, h.n));
  a.n_tiles = (h.n + kTile - 1) / kTile;
  // about 16 waves per CU on 256 CUs, each over a contiguous run of tiles
  const uint64_t max_waves = 256u * 16u;
  const uint64_t waves0 = a.n_tiles < max_waves ? a.n_tiles : max_waves;
  a.tiles_per_wave = (a.n_tiles + waves0 - 1) / waves0;
  const uint64_t waves = (a.n_tiles + a.tiles_per_wave - 1) / a.tiles_per_wave;
  const uint64_t wpb = kBlockThreads / kWave;
  const dim3 grid((unsigned)((waves + wpb - 1) / wpb));
  a.dict = dict_of(&h);
  if (h.layout == WC_LAYOUT_K15)
    hipLaunchKernelGGL(k_decode<WC_LAYOUT_K15>, grid, dim3(kBlockThreads), 0, s, a);
  else
    hipLaunchKernelGGL(k_decode<WC_LAYOUT_BYTESPLIT>, grid, dim3(kBlockThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace wc
