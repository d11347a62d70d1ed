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
template <int LAYOUT, bool SELECT = false>
__device__ inline void build_pair_table(uint32_t* __restrict__ T2, const Dict& d) {
  for (int p = threadIdx.x; p < 256; p += blockDim.x) {
    uint32_t lo, hi;
    if constexpr (SELECT) {
      // the 16 symbols by constant index (scalar loads of the kernel
      // argument) and a select per lane: no vector-memory load, so a wave
      // that has issued global->LDS loads builds its share without waiting
      // for them (the compiler awaits a vector load with vmcnt(0) while
      // such loads are pending)
      lo = 0;
      hi = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        lo = (p & 15) == i ? d.sym[i] : lo;
        hi = (p >> 4) == i ? d.sym[i] : hi;
      }
    } else {
      lo = d.sym[p & 15];
      hi = d.sym[p >> 4];
    }
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
__device__ inline void rebuild_lane(const uint32_t* __restrict__ T2, const Lane4& l,
                                    uint32_t out[16]) {
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) rebuild_group<LAYOUT>(T2, l.codes[k], l.raw[k], out + 4 * k);
}

// Code-15 (escape) marks of the lane's groups: bit 4i + 3 of esc[k] is set
// when weight i of group k escapes (the low three bits of a nibble carry into
// its bit 3 only when they are all set, and bit 3 itself must be set).
// Returns whether the lane has any.
__device__ inline uint32_t nibble15(uint32_t c) {
  return ((c & 0x77777777u) + 0x11111111u) & c & 0x88888888u;
}

__device__ inline bool escape_marks(const Lane4& l, uint32_t esc[kLaneGroups]) {
  uint32_t any = 0;
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    esc[k] = nibble15(l.codes[k]);
    any |= esc[k];
  }
  return any != 0;
}

// The first escape record at or after weight t (count if none), in either
// escape form: a search of the positions (escape_cursor), or, in the
// compact form, which has no positions, the index entry of t's tile plus the
// code-15 marks between the tile start and t, counted by the wave (lane l
// takes weights 32 l .. 32 l + 31 of the tile).  Wave-uniform.
__device__ inline uint64_t escape_cursor_at(bool compact, const uint32_t* __restrict__ idx,
                                            const uint32_t* __restrict__ pos,
                                            const uint8_t* __restrict__ codes, uint64_t count,
                                            uint64_t n, uint64_t t) {
  if (!compact) return escape_cursor(idx, pos, count, n, t);
  if (count == 0 || t >= n) return count;
  const uint64_t j = t / WC_INDEX_TILE;
  uint64_t lo = idx[j];
  lo = lo < count ? lo : count;
  const uint32_t rem = (uint32_t)(t % WC_INDEX_TILE);
  if (rem == 0) return lo;
  const uint32_t lw = 32u * (uint32_t)lane_id();
  uint32_t c = 0;
  if (lw < rem) {
    // 16 aligned bytes of codes: the lane's 32 weights, all before n
    const u32x4 v = *(const u32x4*)(codes + (j * WC_INDEX_TILE + lw) / 2);
    const uint32_t k = rem - lw;  // the lane's weights below t
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t m = nibble15(v[d]);  // bit 4i + 3: weight 8d + i escapes
      const uint32_t w0 = 8u * (uint32_t)d;
      if (w0 >= k)
        m = 0;
      else if (w0 + 8u > k)
        m &= (1u << (4u * (k - w0))) - 1u;
      c += (uint32_t)__popc(m);
    }
  }
  lo += wave_sum_u32(c);
  return lo < count ? lo : count;
}

// Escape count of the lane.
__device__ inline uint32_t count_marks(const uint32_t esc[kLaneGroups]) {
  uint32_t n = 0;
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) n += (uint32_t)__popc(esc[k]);
  return n;
}

// Bit k set when group k holds an escape.
__device__ inline uint32_t group_mask(const uint32_t esc[kLaneGroups]) {
  uint32_t g = 0;
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) g |= (esc[k] ? 1u : 0u) << k;
  return g;
}

// First escape records a tile may need, loaded with the tile's own data so a
// tile with at most 64 escapes waits for no further memory round trip:
// lane l holds record e + l (pos = 0xFFFFFFFF past the end of the stream).
struct EscBatch {
  uint32_t pos;
  uint32_t sym;
};

template <int LAYOUT>
__device__ inline uint32_t load_sym(const uint8_t* __restrict__ esc_sym, uint32_t idx) {
  if (LAYOUT == WC_LAYOUT_BYTESPLIT) return esc_sym[idx];
  return ((const uint16_t*)esc_sym)[idx] & 0x1FFu;
}

// Escape record loads are never skipped: an index past the stream is
// clamped to `last` (n_esc - 1, or 0 with the stream pointers aimed at the
// container header when there are no escapes) and its result discarded, so
// every path issues the same loads and no wait is widened by a branch.
// Record indices and positions fit in 32 bits (n < 2^32).
template <int LAYOUT>
__device__ inline EscBatch load_esc(const uint32_t* __restrict__ esc_pos,
                                    const uint8_t* __restrict__ esc_sym, uint64_t n_esc,
                                    uint64_t last, uint64_t e) {
  const uint32_t idx = (uint32_t)e + (uint32_t)lane_id();
  const bool ok = e + (uint64_t)lane_id() < n_esc;
  const uint32_t ic = ok ? idx : (uint32_t)last;
  const uint32_t p = esc_pos[ic];
  const uint32_t sy = load_sym<LAYOUT>(esc_sym, ic);
  EscBatch b;
  b.pos = ok ? p : 0xFFFFFFFFu;
  b.sym = sy;
  return b;
}

// The stage is accessed with hand-written LDS instructions: the compiler
// would otherwise wait for every outstanding vector-memory operation before
// the first LDS store (it cannot tell the stage apart from the global->LDS
// ring buffers of the decode kernel).  A wave's LDS instructions execute in
// order, so stores are visible to the wave's later loads; loads wait for
// their own data (lgkmcnt) before returning.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// OR one escape symbol into its zero placeholder in the wave's LDS stage.
template <int LAYOUT>
__device__ inline void apply_escape(uint32_t* __restrict__ stage, uint32_t pos, uint32_t sym,
                                    uint64_t tile_start, uint32_t tile_len) {
  // positions are below 2^32; a record past the stream (pos 0xFFFFFFFF) or
  // before the tile wraps to a large offset
  const uint32_t p = pos - (uint32_t)tile_start;
  if (pos != 0xFFFFFFFFu && p < tile_len) {
    const uint32_t v = (sym << (LAYOUT == WC_LAYOUT_K15 ? 7 : 8)) << (16u * (p & 1u));
    asm volatile("ds_or_b32 %0, %1" : : "v"(lds_addr(stage + (p >> 1))), "v"(v) : "memory");
  }
}

// The wave's LDS stage holds one tile in weight order: tile weight p at
// dword p / 2, so lane L's group k (tile group L + 64k) at dwords
// [4 (L + 64k), 4 (L + 64k) + 4).
// Only groups holding an escape (bit k of `gmask`) go through the stage: the
// records patch only those, so the rest stay in registers.
__device__ inline void stage_store(uint32_t* __restrict__ stage, const uint32_t out[16],
                                   uint32_t gmask) {
  const uint32_t base = lds_addr(stage) + 16u * (uint32_t)lane_id();
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    if ((gmask >> k) & 1u) {
      const u32x4 v = {out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]};
      asm volatile("ds_write_b128 %0, %1" : : "v"(base + 1024u * k), "v"(v) : "memory");
    }
  }
}

// All four of the lane's group slots are read at once, behind one wait (one
// LDS round trip instead of one per group); only the staged groups (bit k of
// gmask) are taken.
__device__ inline void stage_load(const uint32_t* __restrict__ stage, uint32_t out[16],
                                  uint32_t gmask) {
  static_assert(kLaneGroups == 4, "four groups per lane");
  const uint32_t base = lds_addr(stage) + 16u * (uint32_t)lane_id();
  u32x4 v[kLaneGroups];
  asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
               "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(base) : "memory");
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    const bool take = (gmask >> k) & 1u;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[4 * k + i] = take ? v[k][i] : out[4 * k + i];
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
      const uint32_t ic = ok ? (uint32_t)idx : (uint32_t)last;
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

// ---- LDS ring of tiles ----------------------------------------------------
//
// A ring slot (4 KB per wave) holds one tile as loaded by global->LDS loads:
// codes at bytes [0, 1024), raw part at [1024, 3072) (K15 uses 1792 bytes),
// and the tile's first 64 escape records at [3072, 3584): positions at
// dwords 768.., and at dwords 832.. the dword holding each symbol (a dense
// tile's symbol run replaces all of it once the tile is in registers).  The
// loads count in vmcnt and the compiler does not track their LDS writes, so
// users await them with explicit counts before reading the slot, and read it
// with hand-written LDS instructions.  Once read, the slot can serve as the
// tile's escape stage.

// 4 KB of tile and records, plus room for a dense tile's symbol run (up to
// 4096 bytes from a 16-byte-aligned start, read back in 20-byte windows).
constexpr uint32_t kRingSlotDwords = 1040;

// ring_wait_ahead: how a ring user awaits its slot.  vmcnt counts every
// outstanding vector-memory operation, but only operations of one kind are
// taken to complete in issue order: global->LDS loads among themselves.
// Ordinary loads and stores may complete before an older global->LDS load
// (the compiler's own wait placement assumes no order between the kinds:
// with one pending it waits for vmcnt(0)).  So "at most N outstanding"
// proves a global->LDS load complete only when N counts global->LDS loads
// issued after it; ordinary loads and stores in between are never counted
// (they only make the wait longer).  The decode issues the next tile's 3
// ring loads after the current tile's record loads and waits for at most
// those 3; the fused GEMV issues a tile's 3 ring loads and its 2 record
// loads (ring_load_esc) together, after the current tile's, and waits for at
// most those 5.
constexpr int kRingAhead = 3;
constexpr int kRingAheadEsc = kRingAhead + 2;

// Tile whose first group is G (a multiple of 256, so every window below is
// 16-byte aligned): 3 instructions.
template <int LAYOUT>
__device__ inline void ring_load_tile(const uint8_t* codes, const uint8_t* raw, uint64_t G,
                                      uint32_t* buf) {
  constexpr uint32_t kRawTile = LAYOUT == WC_LAYOUT_K15 ? 7 * kTile / 8 : kTile;
  const uint32_t lane = (uint32_t)lane_id();
  const uint8_t* cp = codes + 4 * G;
  const uint8_t* rp = raw + (LAYOUT == WC_LAYOUT_K15 ? 7 * G : 8 * G);
  const uint32_t o2 = 1024u + 16u * lane;  // K15: lanes past 1792 bytes re-read the last 16
  lds_dma16(cp + 16 * lane, buf);
  lds_dma16(rp + 16 * lane, buf + 256);
  lds_dma16(rp + (o2 + 16u <= kRawTile ? o2 : kRawTile - 16u), buf + 512);
}

// The slot's tile in the group mapping (lane L: groups L + 64k).
template <int LAYOUT>
__device__ inline void ring_read_tile(const uint32_t* buf, Lane4& l) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const uint32_t lane = (uint32_t)lane_id();
  const uint32_t cb = lds_addr(buf) + 4u * lane;  // code of group L at dword L
  u32x2 c01, c23;
  if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
    const uint32_t rb = lds_addr(buf) + 1024u + 8u * lane;  // raw of group L
    u32x4 r01, r23;
    // outputs early-clobber: the block reads its address registers after
    // writing results
    asm volatile(
        "ds_read2st64_b32 %0, %4 offset1:1\n\t"
        "ds_read2st64_b32 %1, %4 offset0:2 offset1:3\n\t"
        "ds_read2st64_b64 %2, %5 offset1:1\n\t"
        "ds_read2st64_b64 %3, %5 offset0:2 offset1:3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c01), "=&v"(c23), "=&v"(r01), "=&v"(r23)
        : "v"(cb), "v"(rb)
        : "memory");
    l.raw[0][0] = r01[0]; l.raw[0][1] = r01[1]; l.raw[1][0] = r01[2]; l.raw[1][1] = r01[3];
    l.raw[2][0] = r23[0]; l.raw[2][1] = r23[1]; l.raw[3][0] = r23[2]; l.raw[3][1] = r23[3];
  } else {
    // group L + 64k starts at raw byte 7L + 448k: dwords d0 + 112k + {0,1,2}
    const uint32_t byte = 7u * lane, sh = (byte & 3u) * 8u;
    const uint32_t rb = lds_addr(buf) + 1024u + 4u * (byte >> 2);
    uint32_t w[12];
    asm volatile(
        "ds_read2st64_b32 %0, %14 offset1:1\n\t"
        "ds_read2st64_b32 %1, %14 offset0:2 offset1:3\n\t"
        "ds_read_b32 %2, %15\n\t"
        "ds_read_b32 %3, %15 offset:4\n\t"
        "ds_read_b32 %4, %15 offset:8\n\t"
        "ds_read_b32 %5, %15 offset:448\n\t"
        "ds_read_b32 %6, %15 offset:452\n\t"
        "ds_read_b32 %7, %15 offset:456\n\t"
        "ds_read_b32 %8, %15 offset:896\n\t"
        "ds_read_b32 %9, %15 offset:900\n\t"
        "ds_read_b32 %10, %15 offset:904\n\t"
        "ds_read_b32 %11, %15 offset:1344\n\t"
        "ds_read_b32 %12, %15 offset:1348\n\t"
        "ds_read_b32 %13, %15 offset:1352\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c01), "=&v"(c23), "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]),
          "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]), "=&v"(w[7]), "=&v"(w[8]), "=&v"(w[9]),
          "=&v"(w[10]), "=&v"(w[11])
        : "v"(cb), "v"(rb)
        : "memory");
#pragma unroll
    for (int k = 0; k < kLaneGroups; ++k) {
      l.raw[k][0] = __builtin_amdgcn_alignbit(w[3 * k + 1], w[3 * k], sh);
      l.raw[k][1] = __builtin_amdgcn_alignbit(w[3 * k + 2], w[3 * k + 1], sh);
    }
  }
  l.codes[0] = c01[0]; l.codes[1] = c01[1]; l.codes[2] = c23[0]; l.codes[3] = c23[1];
}

// Records e0 .. e0 + 63 (lane j: record e0 + j, clamped to `last` past the
// stream): 2 instructions.
template <int LAYOUT>
__device__ inline void ring_load_esc(const uint32_t* esc_pos, const uint8_t* esc_sym, uint64_t n_esc,
                                     uint64_t last, uint64_t e0, uint32_t* buf) {
  constexpr uint32_t kSymBytes = LAYOUT == WC_LAYOUT_K15 ? 2 : 1;
  const uint64_t idx = e0 + (uint64_t)lane_id();
  const uint32_t ic = idx < n_esc ? (uint32_t)idx : (uint32_t)last;
  lds_dma4(esc_pos + ic, buf + 768);
  lds_dma4(esc_sym + (((uint64_t)ic * kSymBytes) & ~(uint64_t)3), buf + 832);
}

template <int LAYOUT>
__device__ inline EscBatch ring_read_esc(const uint32_t* buf, uint64_t e0, uint64_t n_esc,
                                         uint64_t last) {
  constexpr uint32_t kSymBytes = LAYOUT == WC_LAYOUT_K15 ? 2 : 1;
  const uint32_t ad = lds_addr(buf) + 4u * (uint32_t)lane_id();
  uint32_t p, w;
  asm volatile("ds_read_b32 %0, %2 offset:3072\n\tds_read_b32 %1, %2 offset:3328\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(p), "=&v"(w) : "v"(ad) : "memory");
  const uint64_t idx = e0 + (uint64_t)lane_id();
  const uint32_t ic = idx < n_esc ? (uint32_t)idx : (uint32_t)last;
  EscBatch b;
  b.pos = idx < n_esc ? p : 0xFFFFFFFFu;
  b.sym = (w >> (8u * ((ic * kSymBytes) & 3u))) & (LAYOUT == WC_LAYOUT_K15 ? 0x1FFu : 0xFFu);
  return b;
}

// ---- dense escape tiles: per-group symbol windows -----------------------
//
// When a tile holds more escapes than one wave-wide batch of records, each
// group reads its own records instead: the records are in position order, so
// group g's records start at the tile's first record plus the escape count of
// groups 0 .. g-1 (a prefix sum over the wave), and are consecutive.  The
// group loads that run of symbols as one window and writes the k-th symbol
// into its k-th code-15 weight, all in registers.

// Inclusive prefix sum over the wave: shifts within rows of 16 lanes, then
// the row totals broadcast to the following rows (DPP).
__device__ inline uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Bit i set: weight i of the group has code 15.
__device__ inline uint32_t group_esc_bits(uint32_t c) {
  uint32_t t = nibble15(c) >> 3;  // bit 4i
  t = (t | (t >> 3)) & 0x03030303u;
  t = (t | (t >> 6)) & 0x000F000Fu;
  return (t | (t >> 12)) & 0xFFu;
}

// Ranks of a group's code-15 weights: byte j of rl (rh) = number of code-15
// weights before weight j (4 + j); byte j of ml (mh) = 0xFF when weight j
// (4 + j) has code 15, else 0.
__device__ inline void escape_ranks(uint32_t m, uint32_t& rl, uint32_t& rh, uint32_t& ml,
                                    uint32_t& mh) {
  const uint32_t sl = ((m & 15u) * 0x00204081u) & 0x01010101u;  // byte j = bit j
  const uint32_t sh = (((m >> 4) & 15u) * 0x00204081u) & 0x01010101u;
  const uint32_t il = sl * 0x01010101u;  // inclusive prefix per byte (at most 4: no carries)
  const uint32_t ih = sh * 0x01010101u + (il >> 24) * 0x01010101u;
  rl = il - sl;
  rh = ih - sh;
  ml = sl * 0xFFu;
  mh = sh * 0xFFu;
}

#ifndef WC_WIN_PASS
#define WC_WIN_PASS 4
#endif
constexpr int kWinPass = WC_WIN_PASS;  // groups whose windows are in flight together
#ifndef WC_DENSE_MIN
#define WC_DENSE_MIN 64
#endif
constexpr uint32_t kDenseMin = WC_DENSE_MIN;  // tiles with more escapes take the window path

template <int LAYOUT>
struct WinDwords {
  static constexpr int value = LAYOUT == WC_LAYOUT_K15 ? 5 : 3;  // 8 symbols + alignment
};

// Write group k's symbols (window w, byte offset off of the first symbol)
// into the zero placeholders of its rebuilt weights out[0..3].
template <int LAYOUT>
__device__ inline void expand_window(uint32_t m, const uint32_t (&w)[WinDwords<LAYOUT>::value],
                                     uint32_t off, uint32_t out[4]) {
  constexpr int W = WinDwords<LAYOUT>::value;
  // shift the window so that the first symbol starts at byte 0
  uint32_t d[W];
#pragma unroll
  for (int i = 0; i < W; ++i) d[i] = w[i];
  const uint32_t s = off >> 2, sh = (off & 3u) * 8u;
  if (__ballot(s != 0)) {  // only windows moved back from the stream's end
#pragma unroll
    for (int t = 0; t < W - 1; ++t) {
      const bool mv = s > (uint32_t)t;
#pragma unroll
      for (int i = 0; i < W; ++i) d[i] = mv ? (i + 1 < W ? d[i + 1] : 0u) : d[i];
    }
  }
  uint32_t rl, rh, ml, mh;
  escape_ranks(m, rl, rh, ml, mh);
  if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
    const uint32_t a0 = __builtin_amdgcn_alignbit(d[1], d[0], sh);
    const uint32_t a1 = __builtin_amdgcn_alignbit(d[2], d[1], sh);
    // byte j of hl (hh) = symbol of weight j (4 + j), 0 when it is not an escape
    const uint32_t hl = __builtin_amdgcn_perm(a1, a0, (rl & ml) | (0x0C0C0C0Cu & ~ml));
    const uint32_t hh = __builtin_amdgcn_perm(a1, a0, (rh & mh) | (0x0C0C0C0Cu & ~mh));
    out[0] |= __builtin_amdgcn_perm(0u, hl, 0x010C000Cu);
    out[1] |= __builtin_amdgcn_perm(0u, hl, 0x030C020Cu);
    out[2] |= __builtin_amdgcn_perm(0u, hh, 0x010C000Cu);
    out[3] |= __builtin_amdgcn_perm(0u, hh, 0x030C020Cu);
  } else {
    // symbols 0..7 of the window as little-endian u16 in a[0..3]; their low
    // bytes gathered into lo[0..1] and their high bytes (the symbol's ninth
    // bit) into hi[0..1], so that one byte permute by rank reaches any of
    // the eight, as in the byte-split case
    uint32_t a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __builtin_amdgcn_alignbit(d[i + 1], d[i], sh);
    const uint32_t lo0 = __builtin_amdgcn_perm(a[1], a[0], 0x06040200u);
    const uint32_t lo1 = __builtin_amdgcn_perm(a[3], a[2], 0x06040200u);
    const uint32_t hi0 = __builtin_amdgcn_perm(a[1], a[0], 0x07050301u) & 0x01010101u;
    const uint32_t hi1 = __builtin_amdgcn_perm(a[3], a[2], 0x07050301u) & 0x01010101u;
    // byte j of the selectors = rank of weight j (4 + j), or a zero byte
    const uint32_t sl = (rl & ml) | (0x0C0C0C0Cu & ~ml);
    const uint32_t sh2 = (rh & mh) | (0x0C0C0C0Cu & ~mh);
    const uint32_t l4 = __builtin_amdgcn_perm(lo1, lo0, sl), h4 = __builtin_amdgcn_perm(hi1, hi0, sl);
    const uint32_t l8 = __builtin_amdgcn_perm(lo1, lo0, sh2), h8 = __builtin_amdgcn_perm(hi1, hi0, sh2);
    // weights 2j, 2j+1: their symbols as the two halves of a dword, moved
    // above the 7 mantissa bits
    out[0] |= __builtin_amdgcn_perm(h4, l4, 0x05010400u) << 7;
    out[1] |= __builtin_amdgcn_perm(h4, l4, 0x07030602u) << 7;
    out[2] |= __builtin_amdgcn_perm(h8, l8, 0x05010400u) << 7;
    out[3] |= __builtin_amdgcn_perm(h8, l8, 0x07030602u) << 7;
  }
}

// Per group of the lane: m = its code-15 weights (bit i: weight i), c = their
// count, first = its first record relative to the tile's first (groups
// L + 64k in tile order: all of k = 0, then k = 1, ...; counts are packed two
// per dword for the wave's prefix sum).
__device__ inline void group_records(const Lane4& l, uint32_t m[kLaneGroups],
                                     uint32_t c[kLaneGroups], uint32_t first[kLaneGroups]) {
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    m[k] = group_esc_bits(l.codes[k]);
    c[k] = (uint32_t)__popc(m[k]);
  }
  const uint32_t p01 = c[0] | (c[1] << 16), p23 = c[2] | (c[3] << 16);
  const uint32_t i01 = wave_incl_scan_dpp(p01), i23 = wave_incl_scan_dpp(p23);
  const uint32_t t01 = (uint32_t)__builtin_amdgcn_readlane((int)i01, kWave - 1);
  const uint32_t t23 = (uint32_t)__builtin_amdgcn_readlane((int)i23, kWave - 1);
  const uint32_t x01 = i01 - p01, x23 = i23 - p23;
  first[0] = x01 & 0xFFFFu;
  first[1] = (t01 & 0xFFFFu) + (x01 >> 16);
  first[2] = (t01 & 0xFFFFu) + (t01 >> 16) + (x23 & 0xFFFFu);
  first[3] = (t01 & 0xFFFFu) + (t01 >> 16) + (t23 & 0xFFFFu) + (x23 >> 16);
}

// A dense tile's symbol run (records e .. e + cnt - 1, cnt <= 2048) into a
// ring slot with global->LDS loads: the run's 16-byte chunks from the one
// holding record e's symbol, 64 chunks per instruction (at most 5; chunks
// past the stream's padded end re-read its last one).  Returns the byte
// offset of record e's symbol in the slot.  The caller awaits the loads
// (ring_wait_ahead) before patch_tile_symrun reads the slot.
template <int LAYOUT>
__device__ inline uint32_t ring_load_symrun(const uint8_t* esc_sym, uint64_t sym_last, uint64_t e,
                                            uint32_t cnt, uint32_t* buf) {
  constexpr uint64_t kSymBytes = LAYOUT == WC_LAYOUT_K15 ? 2 : 1;
  const uint64_t b0 = e * kSymBytes;
  const uint64_t base = b0 & ~(uint64_t)15;
  const uint32_t nch = (uint32_t)((b0 + cnt * kSymBytes - base + 15) >> 4);
  const uint64_t last_chunk = (4 * (sym_last + 1) - 16) >> 4;  // the padded extent is 16-byte whole
  const uint32_t lane = (uint32_t)lane_id();
  for (uint32_t c0 = 0; c0 < nch; c0 += kWave) {
    if (c0 + lane < nch) {
      uint64_t ch = (base >> 4) + c0 + lane;
      ch = ch < last_chunk ? ch : last_chunk;
      lds_dma16_keep(esc_sym + 16 * ch, buf + 4 * c0);
    }
  }
  return (uint32_t)(b0 - base);
}

// Compact form (no positions): instead of a tile's first records, the first
// 512 bytes of its symbol run, from the 16-byte chunk that holds record e0,
// go into buf[768 .. 896) with the tile's ring loads: two global->LDS loads,
// as many as ring_load_esc issues, so the ring's waits stay the same.  A
// tile whose symbols fit (kAheadSyms) is patched from there without a load
// of its own.  Without escapes the loads read the stream's first chunk.
constexpr uint32_t kAheadRunBytes = 512;
template <int LAYOUT>
__device__ inline void ring_load_symrun_ahead(const uint8_t* esc_sym, uint64_t sym_last, uint64_t n_esc,
                                              uint64_t e0, uint32_t* buf) {
  constexpr uint64_t kSymBytes = LAYOUT == WC_LAYOUT_K15 ? 2 : 1;
  const uint32_t lane = (uint32_t)lane_id();
  uint64_t c0 = 0, c1 = 0;
  if (n_esc) {
    const uint64_t last_chunk = (4 * (sym_last + 1) - 16) >> 4;  // the padded extent is 16-byte whole
    const uint64_t base = (e0 * kSymBytes) >> 4;
    c0 = base + lane;
    c1 = base + 16 + lane;
    c0 = c0 < last_chunk ? c0 : last_chunk;
    c1 = c1 < last_chunk ? c1 : last_chunk;
  }
  if (lane < 16) {
    lds_dma16_keep(esc_sym + 16 * c0, buf + 768);
    lds_dma16_keep(esc_sym + 16 * c1, buf + 832);
  }
}
template <int LAYOUT>
struct AheadSyms {  // records a prefetched run holds whatever its alignment
  static constexpr uint32_t value = (kAheadRunBytes - 16) / (LAYOUT == WC_LAYOUT_K15 ? 2 : 1);
};

// The windows of four groups (W dwords each, from LDS byte addresses ad[k],
// dword-aligned) behind one wait: one LDS round trip instead of four.
template <int W>
__device__ inline void lds_read_windows4(const uint32_t ad[4], uint32_t (&w)[4][W]) {
  static_assert(W == 3 || W == 5, "window sizes of the two layouts");
  if constexpr (W == 3) {
    asm volatile(
        "ds_read_b32 %0, %12\n\tds_read_b32 %1, %12 offset:4\n\tds_read_b32 %2, %12 offset:8\n\t"
        "ds_read_b32 %3, %13\n\tds_read_b32 %4, %13 offset:4\n\tds_read_b32 %5, %13 offset:8\n\t"
        "ds_read_b32 %6, %14\n\tds_read_b32 %7, %14 offset:4\n\tds_read_b32 %8, %14 offset:8\n\t"
        "ds_read_b32 %9, %15\n\tds_read_b32 %10, %15 offset:4\n\tds_read_b32 %11, %15 offset:8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0][0]), "=&v"(w[0][1]), "=&v"(w[0][2]), "=&v"(w[1][0]), "=&v"(w[1][1]),
          "=&v"(w[1][2]), "=&v"(w[2][0]), "=&v"(w[2][1]), "=&v"(w[2][2]), "=&v"(w[3][0]),
          "=&v"(w[3][1]), "=&v"(w[3][2])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b32 %0, %20\n\tds_read_b32 %1, %20 offset:4\n\tds_read_b32 %2, %20 offset:8\n\t"
        "ds_read_b32 %3, %20 offset:12\n\tds_read_b32 %4, %20 offset:16\n\t"
        "ds_read_b32 %5, %21\n\tds_read_b32 %6, %21 offset:4\n\tds_read_b32 %7, %21 offset:8\n\t"
        "ds_read_b32 %8, %21 offset:12\n\tds_read_b32 %9, %21 offset:16\n\t"
        "ds_read_b32 %10, %22\n\tds_read_b32 %11, %22 offset:4\n\tds_read_b32 %12, %22 offset:8\n\t"
        "ds_read_b32 %13, %22 offset:12\n\tds_read_b32 %14, %22 offset:16\n\t"
        "ds_read_b32 %15, %23\n\tds_read_b32 %16, %23 offset:4\n\tds_read_b32 %17, %23 offset:8\n\t"
        "ds_read_b32 %18, %23 offset:12\n\tds_read_b32 %19, %23 offset:16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0][0]), "=&v"(w[0][1]), "=&v"(w[0][2]), "=&v"(w[0][3]), "=&v"(w[0][4]),
          "=&v"(w[1][0]), "=&v"(w[1][1]), "=&v"(w[1][2]), "=&v"(w[1][3]), "=&v"(w[1][4]),
          "=&v"(w[2][0]), "=&v"(w[2][1]), "=&v"(w[2][2]), "=&v"(w[2][3]), "=&v"(w[2][4]),
          "=&v"(w[3][0]), "=&v"(w[3][1]), "=&v"(w[3][2]), "=&v"(w[3][3]), "=&v"(w[3][4])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  }
}

// Two groups' windows of 5 dwords behind one wait.
__device__ inline void lds_read_windows2(const uint32_t ad[2], uint32_t (&w)[2][5]) {
  asm volatile(
      "ds_read_b32 %0, %10\n\tds_read_b32 %1, %10 offset:4\n\tds_read_b32 %2, %10 offset:8\n\t"
      "ds_read_b32 %3, %10 offset:12\n\tds_read_b32 %4, %10 offset:16\n\t"
      "ds_read_b32 %5, %11\n\tds_read_b32 %6, %11 offset:4\n\tds_read_b32 %7, %11 offset:8\n\t"
      "ds_read_b32 %8, %11 offset:12\n\tds_read_b32 %9, %11 offset:16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0][0]), "=&v"(w[0][1]), "=&v"(w[0][2]), "=&v"(w[0][3]), "=&v"(w[0][4]),
        "=&v"(w[1][0]), "=&v"(w[1][1]), "=&v"(w[1][2]), "=&v"(w[1][3]), "=&v"(w[1][4])
      : "v"(ad[0]), "v"(ad[1])
      : "memory");
}

// A tile's symbol run ahead of its use, in place of its first records:
// the 16-byte chunks from the one holding record e0, as many as `cnt`
// symbols need (the count the escape index gives), at most `max_chunks`
// (<= 128), into the slot from dword 768 on, with the tile's ring loads.  Two
// global->LDS loads, as many as ring_load_esc issues (each with at least one
// lane), so the ring's waits stay the same.  Chunks past the stream's padded
// end re-read its last.  A slot of S bytes holds (S - 3104) / 16 chunks: the
// run's windows (wc_tile patch paths) read up to 20 bytes past its end.
__host__ __device__ constexpr uint32_t run_ahead_syms(uint32_t max_chunks, int layout) {
  // records a run ahead holds whatever its alignment
  return (16u * max_chunks - 16u) / (layout == WC_LAYOUT_K15 ? 2u : 1u);
}
template <int LAYOUT>
__device__ inline void ring_load_run_ahead(const uint8_t* esc_sym, uint64_t sym_last, uint64_t n_esc,
                                           uint64_t e0, uint64_t cnt, uint32_t max_chunks,
                                           uint32_t* buf) {
  constexpr uint64_t kSymBytes = LAYOUT == WC_LAYOUT_K15 ? 2 : 1;
  const uint32_t lane = (uint32_t)lane_id();
  uint64_t base = 0, last_chunk = 0;
  uint32_t nch = 1;
  if (n_esc) {
    last_chunk = (4 * (sym_last + 1) - 16) >> 4;  // the padded extent is 16-byte whole
    const uint64_t b0 = e0 * kSymBytes;
    base = b0 >> 4;
    const uint64_t need = ((b0 & 15u) + (cnt < 4096 ? cnt : 4096) * kSymBytes + 15) >> 4;
    nch = need < max_chunks ? (uint32_t)need : max_chunks;
    nch = nch ? nch : 1u;
  }
  uint64_t c0 = base + lane, c1 = base + kWave + lane;
  c0 = c0 < last_chunk ? c0 : last_chunk;
  c1 = c1 < last_chunk ? c1 : last_chunk;
  if (lane < nch || lane == 0) lds_dma16_keep(esc_sym + 16 * c0, buf + 768);
  if (lane + kWave < nch || lane == 0) lds_dma16_keep(esc_sym + 16 * c1, buf + 1024);
}

// Patch a dense tile from its symbol run in LDS (ring_load_symrun, run byte
// offset off0): each group reads the window that starts at its first record
// (byte-split: the four windows in one LDS round trip; K15, whose windows
// are larger: K15_PASS at a time, fewer where registers are short) and
// writes the symbols into its code-15 weights.
template <int LAYOUT, int K15_PASS = 2>
__device__ inline void patch_tile_symrun(const Lane4& l, uint32_t out[16], const uint32_t* buf,
                                         uint32_t off0) {
  static_assert(K15_PASS == 1 || K15_PASS == 2, "K15 windows per LDS round trip");
  constexpr int W = WinDwords<LAYOUT>::value;
  constexpr uint32_t kSymBytes = LAYOUT == WC_LAYOUT_K15 ? 2 : 1;
  static_assert(kLaneGroups == 4, "four groups per lane");
  uint32_t m[kLaneGroups], c[kLaneGroups], first[kLaneGroups];
  group_records(l, m, c, first);
  uint32_t o[kLaneGroups], ad[kLaneGroups];
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    o[k] = off0 + first[k] * kSymBytes;  // < 16 + 4096: the window stays in the slot
    ad[k] = lds_addr(buf) + (o[k] & ~3u);
  }
  if constexpr (LAYOUT == WC_LAYOUT_BYTESPLIT) {
    uint32_t w[kLaneGroups][W];
    lds_read_windows4<W>(ad, w);
#pragma unroll
    for (int k = 0; k < kLaneGroups; ++k)
      if (c[k]) expand_window<LAYOUT>(m[k], w[k], o[k] & 3u, out + 4 * k);
  } else if constexpr (K15_PASS == 2) {
#pragma unroll
    for (int k0 = 0; k0 < kLaneGroups; k0 += 2) {
      uint32_t w[2][W];
      lds_read_windows2(ad + k0, w);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (c[k0 + u]) expand_window<LAYOUT>(m[k0 + u], w[u], o[k0 + u] & 3u, out + 4 * (k0 + u));
    }
  } else {
#pragma unroll
    for (int k = 0; k < kLaneGroups; ++k) {
      uint32_t w[W];
      asm volatile("ds_read_b32 %0, %5\n\tds_read_b32 %1, %5 offset:4\n\tds_read_b32 %2, %5 offset:8\n\t"
                   "ds_read_b32 %3, %5 offset:12\n\tds_read_b32 %4, %5 offset:16\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]) : "v"(ad[k]) : "memory");
      if (c[k]) expand_window<LAYOUT>(m[k], w, o[k] & 3u, out + 4 * k);
    }
  }
}

// A tile with at most kGatherMax escapes in every lane, patched from its
// symbol run in LDS by rank: the tile's r-th record belongs to its r-th
// code-15 weight in tile order, so a weight's record is its group's first
// record (group_records) plus the code-15 weights before it in the group.
// Each lane reads the symbols of its (at most kGatherMax) escapes from the
// run, byte address `run` of the tile's first symbol, in one LDS round
// trip, then ORs them into its staged groups; the stage is written only
// after the reads have returned, so it may overlap the run.  Per escape this
// is a few instructions where the window path spends about 80 per group of
// a K15 tile whatever its marks.
constexpr int kGatherMax = 4;
template <int LAYOUT>
__device__ inline void patch_tile_gather(uint32_t* __restrict__ stage, uint32_t out[16],
                                         const uint32_t m[kLaneGroups],
                                         const uint32_t first[kLaneGroups], uint32_t run) {
  constexpr uint32_t kSymBytes = LAYOUT == WC_LAYOUT_K15 ? 2 : 1;
  constexpr uint32_t kShift = LAYOUT == WC_LAYOUT_K15 ? 7 : 8;
  constexpr uint32_t kSymMask = LAYOUT == WC_LAYOUT_K15 ? 0x1FFu : 0xFFu;
  const uint32_t lane = (uint32_t)lane_id();
  const uint32_t all = m[0] | (m[1] << 8) | (m[2] << 16) | (m[3] << 24);
  uint32_t left = all;
  uint32_t ad[kGatherMax], dst[kGatherMax], sh[kGatherMax];
  bool ok[kGatherMax];
#pragma unroll
  for (int u = 0; u < kGatherMax; ++u) {
    ok[u] = left != 0;
    const uint32_t b = ok[u] ? (uint32_t)__builtin_ctz(left) : 0u;  // bit 8k + j: weight j of group k
    left &= left - 1u;
    const uint32_t k = b >> 3, j = b & 7u;
    const uint32_t f = k == 0 ? first[0] : k == 1 ? first[1] : k == 2 ? first[2] : first[3];
    const uint32_t below = (all >> (b & ~7u)) & ((1u << j) - 1u);  // code-15 weights before j in k
    ad[u] = run + (f + (uint32_t)__popc(below)) * kSymBytes;
    const uint32_t p = 8u * (lane + (uint32_t)kWave * k) + j;  // weight in the tile
    dst[u] = lds_addr(stage) + 4u * (p >> 1);
    sh[u] = kShift + 16u * (p & 1u);
  }
  uint32_t v[kGatherMax];
  if constexpr (LAYOUT == WC_LAYOUT_K15) {
    asm volatile("ds_read_u16 %0, %4\n\tds_read_u16 %1, %5\n\tds_read_u16 %2, %6\n\t"
                 "ds_read_u16 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
                 : "memory");
  } else {
    asm volatile("ds_read_u8 %0, %4\n\tds_read_u8 %1, %5\n\tds_read_u8 %2, %6\n\t"
                 "ds_read_u8 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
                 : "memory");
  }
  uint32_t gmask = 0;
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) gmask |= (m[k] != 0 ? 1u : 0u) << k;
  stage_store(stage, out, gmask);
  wave_lds_sync();
#pragma unroll
  for (int u = 0; u < kGatherMax; ++u)
    if (ok[u]) {
      const uint32_t w = (v[u] & kSymMask) << sh[u];
      asm volatile("ds_or_b32 %0, %1" : : "v"(dst[u]), "v"(w) : "memory");
    }
  wave_lds_sync();
  stage_load(stage, out, gmask);
  wave_lds_sync();  // the stage is reused by this wave's next tile
}

// Patch a tile from per-group windows.  `e` = index of the tile's first
// record; `sym_last` = last dword of the symbol stream's 16-byte padded
// extent (windows are moved back so they end there; their start may then
// fall in the preceding streams of the container).
template <int LAYOUT>
__device__ inline void patch_tile_windows(const Lane4& l, uint32_t out[16],
                                          const uint8_t* __restrict__ esc_sym, uint64_t sym_last,
                                          uint64_t e) {
  constexpr int W = WinDwords<LAYOUT>::value;
  constexpr uint64_t kSymBytes = LAYOUT == WC_LAYOUT_K15 ? 2 : 1;
  uint32_t m[kLaneGroups], c[kLaneGroups], first[kLaneGroups];
  group_records(l, m, c, first);
  // windows are loaded and applied kWinPass groups at a time (fewer live
  // registers for smaller passes)
#pragma unroll
  for (int k0 = 0; k0 < kLaneGroups; k0 += kWinPass) {
    uint32_t w[kWinPass][W], off[kWinPass];
#pragma unroll
    for (int u = 0; u < kWinPass; ++u) {
      const int k = k0 + u;
      const uint64_t byte = (e + first[k]) * kSymBytes;
      int64_t b = (int64_t)(byte >> 2);
      const int64_t bmax = (int64_t)sym_last - (W - 1);
      b = b < bmax ? b : bmax;
      off[u] = (uint32_t)(byte - 4 * (uint64_t)b);
      if (c[k]) {
        const uint32_t* sp = (const uint32_t*)esc_sym + b;
        if constexpr (W == 3) {
          typedef uint32_t u32x3a4 __attribute__((ext_vector_type(3), aligned(4)));
          const u32x3a4 v = *(const u32x3a4*)sp;
          w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2];
        } else {
          typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
          const u32x4a4 v = *(const u32x4a4*)sp;
          w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
          w[u][W - 1] = sp[W - 1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kWinPass; ++u)
      if (c[k0 + u]) expand_window<LAYOUT>(m[k0 + u], w[u], off[u], out + 4 * (k0 + u));
  }
}

}  // namespace wc
