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
// Tile = 2048 consecutive weights handled by one wave: 256 groups of 8
// weights; lane L owns groups L, L+64, L+128 and L+192.  With that mapping
// every stream is read and written in whole lines by each instruction:
// codes 4 bytes per group (256 B contiguous per instruction), byte-split low
// bytes 8 bytes per group (512 B), BF16 output and x 16 bytes per group
// (1 KB); K15 mantissas are 7 bytes per group, read as a 3-dword window.
// A rebuilt group = 4 dwords, dword j holding weights 2j (low half) and
// 2j+1 (high half), which is also the operand layout of v_dot2_f32_bf16.
#pragma once

#include "wc_common.h"

namespace wc {

constexpr int kGroup = 8;                             // weights per group
constexpr int kLaneGroups = kTile / kGroup / kWave;   // groups per lane per tile (4)
constexpr int kStageDwords = kTile / 2;             // per-wave LDS stage: one rebuilt tile

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

// A lane's share of one tile: 4 groups of 8 coded weights.
struct Lane4 {
  uint32_t codes[kLaneGroups];   // group k: 8 codes, weight 8g+i in nibble i
  uint32_t raw[kLaneGroups][2];  // byte-split: 8 low bytes; K15: 56 mantissa bits
};

// The streams of one tile, positioned at its first group G (weights from
// 8G): wave-uniform base pointers that lanes offset by 32-bit group indices,
// which lets loads use a scalar base plus a 32-bit vector offset.
struct GroupBase {
  const uint32_t* codes;  // code dword of group G
  const uint8_t* raw;     // byte-split: low bytes of group G; K15: the dword holding bit 56G
  uint32_t skew;          // K15: (7G) mod 4, the byte offset of group G in that dword
  uint32_t raw_lim;       // K15: last dword of the raw stream's padded extent, from `raw`
};

__device__ inline GroupBase group_base(int layout, const uint8_t* codes, const uint8_t* raw,
                                       uint64_t G, uint64_t raw_last) {
  GroupBase b;
  b.codes = (const uint32_t*)codes + G;
  if (layout == WC_LAYOUT_BYTESPLIT) {
    b.raw = raw + 8u * G;
    b.skew = 0;
    b.raw_lim = 0;
  } else {
    const uint64_t d = (7u * G) >> 2;
    b.raw = raw + 4u * d;
    b.skew = (uint32_t)((7u * G) & 3u);
    b.raw_lim = (uint32_t)(raw_last - d);
  }
  return b;
}

// Group G + lg.  A K15 group's 7 bytes lie in the 3 dwords that start at
// the dword holding its first byte, read with one 12-byte load; near the
// stream's end that window is moved back so it ends inside the stream's
// 16-byte padded extent (the group's bytes then start one or two dwords
// later in it, and only those inside the stream are used).
template <int LAYOUT>
__device__ inline void load_group(const GroupBase& b, uint32_t lg, uint32_t& c, uint32_t r[2]) {
  c = __builtin_nontemporal_load(b.codes + lg);
  if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)b.raw + lg);
    r[0] = v[0];
    r[1] = v[1];
  } else {
    typedef uint32_t u32x3a4 __attribute__((ext_vector_type(3), aligned(4)));
    const uint32_t byte = b.skew + 7u * lg, d = byte >> 2, sh = (byte & 3u) * 8u;
    const int32_t dc = (int32_t)d + 2 <= (int32_t)b.raw_lim ? (int32_t)d : (int32_t)b.raw_lim - 2;
    const u32x3a4 v = __builtin_nontemporal_load((const u32x3a4*)((const uint32_t*)b.raw + dc));
    // the group's first byte sits in window dword d - dc (0, or 1..2 when the
    // window was moved back; then only bytes inside the stream are used)
    const uint32_t mv = (uint32_t)((int32_t)d - dc);
    const uint32_t w0 = mv == 0 ? v[0] : (mv == 1 ? v[1] : v[2]);
    const uint32_t w1 = mv == 0 ? v[1] : (mv == 1 ? v[2] : 0u);
    const uint32_t w2 = mv == 0 ? v[2] : 0u;
    r[0] = __builtin_amdgcn_alignbit(w1, w0, sh);
    r[1] = __builtin_amdgcn_alignbit(w2, w1, sh);
  }
}

#ifndef WC_REBUILD_VALU
#define WC_REBUILD_VALU 0
#endif

// Four codes (one per byte, 0..15) -> the four bytes `tab` holds for them.
// v_perm_b32 picks bytes 0-7 of a register pair by a 3-bit selector, so
// codes 0-7 and 8-15 are looked up separately and merged per byte on code
// bit 3 (selector 12 gives 0x00 and 13 gives 0xFF, which builds the mask).
__device__ inline uint32_t lookup4(const uint32_t tab[4], uint32_t sel, uint32_t mask) {
  const uint32_t a = __builtin_amdgcn_perm(tab[1], tab[0], sel);
  const uint32_t b = __builtin_amdgcn_perm(tab[3], tab[2], sel);
  return (b & mask) | (a & ~mask);
}

__device__ inline void sel_mask(uint32_t c4, uint32_t& sel, uint32_t& mask) {
  sel = c4 & 0x07070707u;
  mask = __builtin_amdgcn_perm(0u, 0u, ((c4 >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
}

// Rebuild one group from registers only: the dictionary bytes come from the
// kernel arguments (SGPRs), no LDS table.
template <int LAYOUT>
__device__ inline void rebuild_group_valu(const Dict& d, uint32_t c, const uint32_t r[2],
                                          uint32_t out[4]) {
  const uint32_t ev = c & 0x0F0F0F0Fu;         // codes of weights 0, 2, 4, 6
  const uint32_t od = (c >> 4) & 0x0F0F0F0Fu;  // codes of weights 1, 3, 5, 7
  const uint32_t c03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);  // codes 0..3 in bytes
  const uint32_t c47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);  // codes 4..7
  uint32_t s0, m0, s1, m1;
  sel_mask(c03, s0, m0);
  sel_mask(c47, s1, m1);
  const uint32_t h03 = lookup4(d.hi, s0, m0), h47 = lookup4(d.hi, s1, m1);
  if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
    // [low(2j), high(2j), low(2j+1), high(2j+1)]
    out[0] = __builtin_amdgcn_perm(h03, r[0], 0x05010400u);
    out[1] = __builtin_amdgcn_perm(h03, r[0], 0x07030602u);
    out[2] = __builtin_amdgcn_perm(h47, r[1], 0x05010400u);
    out[3] = __builtin_amdgcn_perm(h47, r[1], 0x07030602u);
  } else {
    const uint32_t l03 = lookup4(d.lo, s0, m0), l47 = lookup4(d.lo, s1, m1);
    const uint32_t f[4] = {r[0], r[0] >> 14, __builtin_amdgcn_alignbit(r[1], r[0], 28), r[1] >> 10};
    out[0] = __builtin_amdgcn_perm(h03, l03, 0x05010400u) | (f[0] & 0x7Fu) | ((f[0] << 9) & 0x007F0000u);
    out[1] = __builtin_amdgcn_perm(h03, l03, 0x07030602u) | (f[1] & 0x7Fu) | ((f[1] << 9) & 0x007F0000u);
    out[2] = __builtin_amdgcn_perm(h47, l47, 0x05010400u) | (f[2] & 0x7Fu) | ((f[2] << 9) & 0x007F0000u);
    out[3] = __builtin_amdgcn_perm(h47, l47, 0x07030602u) | (f[3] & 0x7Fu) | ((f[3] << 9) & 0x007F0000u);
  }
}

// Rebuild one group into out[4] (escapes carry a zero symbol).
template <int LAYOUT>
__device__ inline void rebuild_group(const uint32_t* __restrict__ T2, uint32_t c, const uint32_t r[2],
                                     uint32_t out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // weights 2j, 2j+1 of the group
    const uint32_t t = T2[(c >> (8 * j)) & 0xFFu];
    if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
      // bytes [low(2j), sym(2j), low(2j+1), sym(2j+1)] from t and the raw dword
      out[j] = __builtin_amdgcn_perm(t, r[j >> 1], (j & 1) ? 0x07030502u : 0x07010500u);
    } else {
      // the pair's 14 mantissa bits sit at bit 14j of the group's 56 bits
      uint32_t f;
      if (j == 0) f = r[0];
      else if (j == 1) f = r[0] >> 14;
      else if (j == 2) f = __builtin_amdgcn_alignbit(r[1], r[0], 28);
      else f = r[1] >> 10;
      out[j] = t | (f & 0x7Fu) | ((f << 9) & 0x007F0000u);
    }
  }
}

template <int LAYOUT>
__device__ inline void rebuild_lane(const uint32_t* __restrict__ T2, const Dict& d, const Lane4& l,
                                    uint32_t out[16]) {
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
#if WC_REBUILD_VALU
    rebuild_group_valu<LAYOUT>(d, l.codes[k], l.raw[k], out + 4 * k);
#else
    rebuild_group<LAYOUT>(T2, l.codes[k], l.raw[k], out + 4 * k);
#endif
  }
}

// Code-15 (escape) marks of the lane's groups: bit 4i of esc[k] is set when
// weight i of group k escapes.  Returns whether the lane has any.
__device__ inline bool escape_marks(const Lane4& l, uint32_t esc[kLaneGroups]) {
  uint32_t any = 0;
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    const uint32_t w = l.codes[k];
    esc[k] = w & (w >> 1) & (w >> 2) & (w >> 3) & 0x11111111u;
    any |= esc[k];
  }
  return any != 0;
}

// Escape count of the lane, and in *gmask bit k set when group k holds one.
__device__ inline uint32_t count_marks(const uint32_t esc[kLaneGroups], uint32_t* gmask) {
  uint32_t n = 0, g = 0;
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    n += __popc(esc[k]);
    g |= (esc[k] ? 1u : 0u) << k;
  }
  *gmask = g;
  return n;
}

// First escape records a tile may need, loaded with the tile's own data so a
// tile with at most 64 escapes waits for no further memory round trip:
// lane l holds record e + l (pos = 0xFFFFFFFF past the end of the stream).
struct EscBatch {
  uint32_t pos;
  uint32_t sym;
};

template <int LAYOUT>
__device__ inline uint32_t load_sym(const uint8_t* __restrict__ esc_sym, uint64_t idx) {
  if (LAYOUT == WC_LAYOUT_BYTESPLIT) return esc_sym[idx];
  return ((const uint16_t*)esc_sym)[idx] & 0x1FFu;
}

// Escape record loads are never skipped: an index past the stream is
// clamped to `last` (n_esc - 1, or 0 with the stream pointers aimed at the
// container header when there are no escapes) and its result discarded, so
// every path issues the same loads and no wait is widened by a branch.
template <int LAYOUT>
__device__ inline EscBatch load_esc(const uint32_t* __restrict__ esc_pos,
                                    const uint8_t* __restrict__ esc_sym, uint64_t n_esc,
                                    uint64_t last, uint64_t e) {
  const uint64_t idx = e + (uint64_t)lane_id();
  const bool ok = idx < n_esc;
  const uint64_t ic = ok ? idx : last;
  const uint32_t p = esc_pos[ic];
  const uint32_t sy = load_sym<LAYOUT>(esc_sym, ic);
  EscBatch b;
  b.pos = ok ? p : 0xFFFFFFFFu;
  b.sym = sy;
  return b;
}

// OR one escape symbol into its zero placeholder in the wave's LDS stage.
template <int LAYOUT>
__device__ inline void apply_escape(uint32_t* __restrict__ stage, uint32_t pos, uint32_t sym,
                                    uint64_t tile_start, uint32_t tile_len) {
  const uint64_t p = (uint64_t)pos - tile_start;  // wraps when before the tile
  if (p < tile_len) {
    const uint32_t v = (sym << (LAYOUT == WC_LAYOUT_K15 ? 7 : 8)) << (16u * (uint32_t)(p & 1u));
    atomicOr(stage + (p >> 1), v);
  }
}

// The wave's LDS stage holds one tile in weight order: tile weight p at
// dword p / 2, so lane L's group k (tile group L + 64k) at dwords
// [4 (L + 64k), 4 (L + 64k) + 4).
// Only groups holding an escape (bit k of `gmask`) go through the stage: the
// records patch only those, so the rest stay in registers.
__device__ inline void stage_store(uint32_t* __restrict__ stage, const uint32_t out[16],
                                   uint32_t gmask) {
  u32x4* st = (u32x4*)stage + lane_id();
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k)
    if ((gmask >> k) & 1u) st[kWave * k] = u32x4{out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]};
}

__device__ inline void stage_load(const uint32_t* __restrict__ stage, uint32_t out[16],
                                  uint32_t gmask) {
  const u32x4* st = (const u32x4*)stage + lane_id();
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    if ((gmask >> k) & 1u) {
      const u32x4 v = st[kWave * k];
      out[4 * k] = v[0]; out[4 * k + 1] = v[1]; out[4 * k + 2] = v[2]; out[4 * k + 3] = v[3];
    }
  }
}

// Apply the tile's escapes to the staged tile: each escape record in
// [e0, e0 + cnt) whose position falls in [tile_start, tile_start + tile_len)
// ORs its symbol into the zero placeholder.  Records are spread across lanes,
// so dense escape runs stay parallel and coalesced: the first 64 come
// preloaded in `first`, the rest in batches of 512 whose loads are all issued
// before any is used.  Call between wave_lds_sync()s.
template <int LAYOUT>
__device__ inline void patch_stage(uint32_t* __restrict__ stage,
                                   const uint32_t* __restrict__ esc_pos,
                                   const uint8_t* __restrict__ esc_sym, uint64_t n_esc,
                                   uint64_t last, uint64_t e0, uint32_t cnt, uint64_t tile_start,
                                   uint32_t tile_len, const EscBatch& first) {
  constexpr int kBatch = 8;
  const int lane = lane_id();
  if ((uint32_t)lane < cnt) apply_escape<LAYOUT>(stage, first.pos, first.sym, tile_start, tile_len);
  for (uint32_t j0 = kWave; j0 < cnt; j0 += kWave * kBatch) {
    uint32_t pos[kBatch], sym[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t j = j0 + (uint32_t)(u * kWave + lane);
      const uint64_t idx = e0 + j;
      const bool ok = j < cnt && idx < n_esc;
      const uint64_t ic = ok ? idx : last;
      const uint32_t p = esc_pos[ic];
      sym[u] = load_sym<LAYOUT>(esc_sym, ic);
      pos[u] = ok ? p : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) apply_escape<LAYOUT>(stage, pos[u], sym[u], tile_start, tile_len);
  }
}

// Registers -> stage -> escapes -> registers (used where the rebuilt tile
// is consumed in registers, as in the GEMV).
template <int LAYOUT>
__device__ inline void patch_tile(uint32_t* __restrict__ stage, uint32_t out[16], uint32_t gmask,
                                  const uint32_t* __restrict__ esc_pos,
                                  const uint8_t* __restrict__ esc_sym, uint64_t n_esc,
                                  uint64_t last, uint64_t e0, uint32_t cnt, uint64_t tile_start,
                                  uint32_t tile_len, const EscBatch& first) {
  stage_store(stage, out, gmask);
  wave_lds_sync();
  patch_stage<LAYOUT>(stage, esc_pos, esc_sym, n_esc, last, e0, cnt, tile_start, tile_len, first);
  wave_lds_sync();
  stage_load(stage, out, gmask);
  wave_lds_sync();  // the stage is reused by this wave's next tile
}

}  // namespace wc
