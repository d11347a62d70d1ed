// wc_tile.h — rebuilding BF16 weights in registers, 32 weights per lane.
//
// The rebuild follows the two layouts of page "Prueba de GLM-5.2 reduce la
// memoria BF16 en casi un 25%", section "Cómo funciona la compresión":
// byte-split puts the dictionary symbol (sign + exponent[7:1]) in the high
// byte over the stored low byte; K15 puts the 9-bit symbol (sign + exponent)
// above the stored 7-bit mantissa.  Escapes (code 15) first come out with a
// zero symbol and are then patched from the exact escape stream.  Rebuilt
// weights stay in registers for the GEMV, as page "Compresión de pesos LLM
// sin pérdida vs 8-bit GGUF: ¿qué está listo para producción?", section
// "¿Qué significa “sin pérdida” para los pesos de un LLM?", describes.
//
// Lane chunk = 32 consecutive weights: 16 bytes of codes, 32 bytes of low
// bytes (byte-split) or 28 bytes = 7 dwords of mantissa bits (K15).  Output
// = 16 dwords, dword j holding weights 2j (low half) and 2j+1 (high half),
// which is also the operand layout of v_dot2_f32_bf16.
#pragma once

#include "wc_common.h"

namespace wc {

// Pair table in LDS: entry p, a byte of the code stream (low nibble = even
// weight, high nibble = odd weight), holds both weights' symbol bits already
// in place in a BF16 pair.  Slot 15 of the dictionary is 0 (escape
// placeholder).
template <int LAYOUT>
__device__ inline void build_pair_table(uint32_t* __restrict__ T2, const Dict& d) {
  for (int p = threadIdx.x; p < 256; p += blockDim.x) {
    const uint32_t lo = d.sym[p & 15], hi = d.sym[p >> 4];
    T2[p] = LAYOUT == WC_LAYOUT_K15 ? (lo << 7) | (hi << 23) : (lo << 8) | (hi << 24);
  }
}

struct Chunk {
  u32x4 codes;
  uint32_t raw[8];  // byte-split: 8 dwords of low bytes; K15: 7 dwords of mantissa bits
};

template <int LAYOUT>
__device__ inline void load_chunk_full(const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ raw, uint64_t chunk,
                                       Chunk& c) {
  c.codes = __builtin_nontemporal_load((const u32x4*)(codes + 16u * chunk));
  if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
    const u32x4 a = __builtin_nontemporal_load((const u32x4*)(raw + 32u * chunk));
    const u32x4 b = __builtin_nontemporal_load((const u32x4*)(raw + 32u * chunk + 16u));
    c.raw[0] = a[0]; c.raw[1] = a[1]; c.raw[2] = a[2]; c.raw[3] = a[3];
    c.raw[4] = b[0]; c.raw[5] = b[1]; c.raw[6] = b[2]; c.raw[7] = b[3];
  } else {
    const uint32_t* r = (const uint32_t*)(raw + 28u * chunk);
#pragma unroll
    for (int k = 0; k < 7; ++k) c.raw[k] = __builtin_nontemporal_load(r + k);
    c.raw[7] = 0;
  }
}

// The tensor's last chunk when n is not a multiple of 32: `valid` weights
// (1..31).  Reads stop at the end of each stream's 16-byte padded extent
// (which always holds whole dwords), and codes of missing weights are cleared
// so they count as neither weights nor escapes.
template <int LAYOUT>
__device__ inline void load_chunk_partial(const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ raw, uint64_t chunk,
                                          uint32_t valid, uint64_t raw_padded, Chunk& c) {
  c.codes = *(const u32x4*)(codes + 16u * chunk);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int nib = (int)valid - 8 * q;
    const uint32_t m = nib >= 8 ? 0xFFFFFFFFu : (nib <= 0 ? 0u : ((1u << (4 * nib)) - 1u));
    c.codes[q] &= m;
  }
  const uint64_t base = (LAYOUT == WC_LAYOUT_K15 ? 28u : 32u) * chunk;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint64_t off = base + 4u * (uint64_t)k;
    const bool in = (LAYOUT == WC_LAYOUT_BYTESPLIT || k < 7) && off + 4u <= raw_padded;
    c.raw[k] = in ? *(const uint32_t*)(raw + off) : 0u;
  }
}

// Rebuild 32 weights into out[16] (escapes carry a zero symbol).
template <int LAYOUT>
__device__ inline void rebuild_chunk(const uint32_t* __restrict__ T2, const Chunk& c,
                                     uint32_t out[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = c.codes[q];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 4 * q + k;  // weights 2j, 2j+1
      const uint32_t t = T2[(w >> (8 * k)) & 0xFFu];
      if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
        // bytes [low(2j), sym(2j), low(2j+1), sym(2j+1)] from t and the raw dword
        const uint32_t L = c.raw[j >> 1];
        out[j] = __builtin_amdgcn_perm(t, L, (j & 1) ? 0x07030502u : 0x07010500u);
      } else {
        // 14 mantissa bits of the pair at bit 14j of the lane's 224-bit window
        const int bit = 14 * j, d = bit >> 5, s = bit & 31;
        uint32_t f;
        if (s + 14 <= 32)
          f = c.raw[d] >> s;
        else
          f = __builtin_amdgcn_alignbit(c.raw[d + 1], c.raw[d], s);
        out[j] = t | (f & 0x7Fu) | ((f << 9) & 0x007F0000u);
      }
    }
  }
}

// Apply the tile's escapes.  The wave's rebuilt chunks go to its LDS stage
// (lane L's weights at dwords [16L, 16L+16)); each escape record in
// [e0, e0 + cnt) whose position falls in [tile_start, tile_start + tile_len)
// ORs its symbol into the zero placeholder; lanes then read their chunks
// back.  Records are spread across lanes, so dense escape runs stay parallel
// and coalesced.
template <int LAYOUT>
__device__ inline void patch_tile(uint32_t* __restrict__ stage, uint32_t out[16],
                                  const uint32_t* __restrict__ esc_pos,
                                  const uint8_t* __restrict__ esc_sym, uint64_t n_esc,
                                  uint64_t e0, uint32_t cnt, uint64_t tile_start,
                                  uint32_t tile_len) {
  const int lane = lane_id();
  u32x4* st = (u32x4*)(stage + 16 * lane);
#pragma unroll
  for (int k = 0; k < 4; ++k) st[k] = u32x4{out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]};
  wave_lds_sync();
  for (uint32_t j = (uint32_t)lane; j < cnt; j += kWave) {
    const uint64_t idx = e0 + j;
    if (idx >= n_esc) break;
    const uint64_t p = (uint64_t)esc_pos[idx] - tile_start;  // wraps when before the tile
    if (p < tile_len) {
      uint32_t s;
      if (LAYOUT == WC_LAYOUT_BYTESPLIT)
        s = esc_sym[idx];
      else
        s = ((const uint16_t*)esc_sym)[idx] & 0x1FFu;
      const uint32_t v = (s << (LAYOUT == WC_LAYOUT_K15 ? 7 : 8)) << (16u * (uint32_t)(p & 1u));
      atomicOr(stage + (p >> 1), v);
    }
  }
  wave_lds_sync();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4 v = st[k];
    out[4 * k] = v[0]; out[4 * k + 1] = v[1]; out[4 * k + 2] = v[2]; out[4 * k + 3] = v[3];
  }
  wave_lds_sync();  // the stage is reused by this wave's next tile
}

}  // namespace wc
