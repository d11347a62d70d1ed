// wc_common.h — library-internal definitions shared by the HIP kernels and
// the C-ABI layer of libwc (gfx950, wave64).
//
// Container layout and symbol definitions follow include/wc.h, which cites
// the pages: "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%",
// section "Cómo funciona la compresión" (byte-split and K15 layouts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wc.h"

namespace wc {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kChunk = 32;             // weights per lane per tile
constexpr int kTile = kWave * kChunk;  // weights per wave per step (2048)
constexpr int kBlockThreads = 256;     // 4 waves per workgroup
constexpr int kPackBlock = kBlockThreads * kChunk;  // weights per encode block (8192)

// ---- container geometry (host + device) ---------------------------------

__host__ __device__ inline uint64_t pad16(uint64_t x) { return (x + 15u) & ~uint64_t(15); }
__host__ __device__ inline int sym_shift(int layout) { return layout == WC_LAYOUT_K15 ? 7 : 8; }
__host__ __device__ inline uint64_t raw_bytes(int layout, uint64_t n) {
  return layout == WC_LAYOUT_K15 ? (7u * n + 7u) / 8u : (layout == WC_LAYOUT_RAW ? 2u * n : n);
}
__host__ __device__ inline uint64_t code_bytes(int layout, uint64_t n) {
  return layout == WC_LAYOUT_RAW ? 0u : (n + 1u) / 2u;
}
__host__ __device__ inline uint64_t sym_bytes(int layout) { return layout == WC_LAYOUT_K15 ? 2u : 1u; }

// Escape-index entries: one per WC_INDEX_TILE-weight tile start plus the
// closing one, none without escapes.
__host__ __device__ inline uint64_t index_entries(uint64_t n, uint64_t n_esc) {
  return n_esc ? (n + WC_INDEX_TILE - 1u) / WC_INDEX_TILE + 1u : 0u;
}

struct Geometry {
  uint64_t off_codes, off_raw, off_esc_pos, off_esc_sym, off_esc_idx, total;
};

// Bytes of the escape-position stream: none in the compact form.
__host__ __device__ inline uint64_t pos_bytes(uint32_t flags, uint64_t n_esc) {
  return (flags & WC_FLAG_COMPACT) ? 0u : 4u * n_esc;
}

__host__ __device__ inline Geometry geometry(int layout, uint64_t n, uint64_t n_esc,
                                             uint32_t flags = 0) {
  Geometry g;
  g.off_codes = WC_HEADER_BYTES;
  g.off_raw = pad16(g.off_codes + code_bytes(layout, n));
  g.off_esc_pos = pad16(g.off_raw + raw_bytes(layout, n));
  g.off_esc_sym = pad16(g.off_esc_pos + pos_bytes(flags, n_esc));
  g.off_esc_idx = pad16(g.off_esc_sym + sym_bytes(layout) * n_esc);
  g.total = pad16(g.off_esc_idx + 4u * index_entries(n, n_esc));
  return g;
}

// Dictionary as kernel argument: symbol per code, slot 15 (escape) = 0, so a
// rebuilt escape holds only its raw bits until it is patched.
struct Dict {
  uint16_t sym[16];
  uint32_t n_dict;
};

// ---- wave primitives -----------------------------------------------------

__device__ inline int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Index of this wave in its workgroup, as a scalar (wave-uniform) value, so
// everything derived from it (tile and row numbers, loop bounds) stays in
// SGPRs and its branches are uniform.
__device__ inline int wave_in_block() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

__device__ inline uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ inline float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Exclusive prefix sum across the wave.
__device__ inline uint32_t wave_excl_scan_u32(uint32_t v) {
  const int lane = lane_id();
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x - v;
}

// Orders this wave's LDS accesses across lanes.  The LDS unit executes one
// wave's instructions in issue order, so only the compiler must be kept from
// moving memory accesses across this point: wavefront-scope fences emit no
// wait (a workgroup-scope fence would also wait for every global load in
// flight, including the next tile's prefetch).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over the wave (DPP shifts within rows of 16 lanes, row totals
// broadcast to the following rows, result read from the last lane).
__device__ inline uint32_t wave_total(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// First index i in [lo, hi) with pos[i] >= t (hi if none), found by the
// whole wave: each round probes 64 entries and keeps the one interval that
// can hold the answer.  Every round shrinks the interval, so it ends even on
// an unsorted (corrupt) array.  Result is wave-uniform.
__device__ inline uint64_t wave_lower_bound(const uint32_t* __restrict__ pos, uint64_t lo,
                                            uint64_t hi, uint64_t t) {
  const int lane = lane_id();
  while (hi - lo > (uint64_t)kWave) {
    const uint64_t step = (hi - lo + kWave - 1) / kWave;
    const uint64_t idx = lo + (uint64_t)lane * step;
    const bool below = idx < hi && (uint64_t)pos[idx] < t;
    const uint64_t k = (uint64_t)__popcll(__ballot(below));
    if (k == 0) return lo;
    const uint64_t nlo = lo + (k - 1) * step + 1;
    const uint64_t nhi = lo + k * step;
    lo = nlo;
    hi = nhi < hi ? nhi : hi;
  }
  const uint64_t idx = lo + (uint64_t)lane;
  const bool below = idx < hi && (uint64_t)pos[idx] < t;
  return lo + (uint64_t)__popcll(__ballot(below));
}

// The first escape record at or after weight t (count if none) of a tensor
// of n weights with `count` records.  The escape index holds the answer for
// every multiple of WC_INDEX_TILE, so a tile start costs one load; any other
// t is searched for among the records of its index tile only.  Entries are
// clamped to [0, count] and to each other, so a corrupt index still gives a
// cursor in range.  Wave-uniform.
__device__ inline uint64_t escape_cursor(const uint32_t* __restrict__ idx,
                                         const uint32_t* __restrict__ pos, uint64_t count,
                                         uint64_t n, uint64_t t) {
  if (count == 0 || t >= n) return count;
  const uint64_t j = t / WC_INDEX_TILE;
  uint64_t lo = idx[j];
  lo = lo < count ? lo : count;
  if (t % WC_INDEX_TILE == 0) return lo;
  uint64_t hi = idx[j + 1];
  hi = hi < lo ? lo : (hi > count ? count : hi);
  return wave_lower_bound(pos, lo, hi, t);
}

// ---- global -> LDS loads and explicit waits --------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void glb_void_t;

// 16 bytes per lane from `src` (per lane) into LDS at dst + 16 * lane (dst
// wave-uniform).  Completion is counted by vmcnt; the compiler does not
// track the LDS write, so readers wait explicitly (wait_vm).  lds_dma16
// marks the load non-temporal (cache policy bit 1): a tile's codes and raw
// part are read once, and so leave the caches to what is reused (x).
// Measured on 6144 x 24576: batch-1 fused GEMV 51.9 -> 50.2 us byte-split,
// 60.9 -> 58.8 K15; decode 91.5 -> 87.3 us K15.  lds_dma16_keep keeps the
// default policy, for data that other waves read again: x, and symbol runs,
// whose first and last 16-byte chunks the neighbouring tiles load too (taken
// non-temporal, the compact-form decode of 4096 x 4096 went from 10.9 to
// 15.9 us).
__device__ inline void lds_dma16(const void* src, uint32_t* dst) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 2);
}
__device__ inline void lds_dma16_keep(const void* src, uint32_t* dst) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}

// 4 bytes per lane into LDS at dst + 4 * lane.
__device__ inline void lds_dma4(const void* src, uint32_t* dst) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 4, 0, 0);
}

// s_waitcnt vmcnt(N) (other counters left alone), N <= 63.
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// s_waitcnt lgkmcnt(0).
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ---- host-side checks ----------------------------------------------------

// WC_OK when *h is exactly the header the format defines for its fields.
inline int validate_header(const wc_header* h) {
  if (h->magic != WC_MAGIC || h->version != WC_VERSION) return WC_E_CORRUPT;
  if (h->layout != WC_LAYOUT_BYTESPLIT && h->layout != WC_LAYOUT_K15 && h->layout != WC_LAYOUT_RAW)
    return WC_E_CORRUPT;
  if (h->n_dict > 15) return WC_E_CORRUPT;
  if (h->layout == WC_LAYOUT_RAW && (h->n_dict != 0 || h->n_esc != 0)) return WC_E_CORRUPT;
  if (h->flags != 0 && (h->flags != WC_FLAG_COMPACT || h->layout == WC_LAYOUT_RAW))
    return WC_E_CORRUPT;
  if (h->n >= (1ull << 32) || h->n_esc > h->n) return WC_E_CORRUPT;
  const uint32_t nsym = h->layout == WC_LAYOUT_K15 ? 512u : 256u;
  for (int k = 0; k < 16; ++k) {
    if (k >= h->n_dict) {
      if (h->dict[k] != 0) return WC_E_CORRUPT;
      continue;
    }
    if (h->dict[k] >= nsym) return WC_E_CORRUPT;
    for (int j = 0; j < k; ++j)
      if (h->dict[j] == h->dict[k]) return WC_E_CORRUPT;
  }
  const Geometry g = geometry(h->layout, h->n, h->n_esc, h->flags);
  if (h->off_codes != g.off_codes || h->off_raw != g.off_raw || h->off_esc_pos != g.off_esc_pos ||
      h->off_esc_sym != g.off_esc_sym || h->off_esc_idx != g.off_esc_idx || h->total_bytes != g.total)
    return WC_E_CORRUPT;
  for (int k = 0; k < 23; ++k)
    if (h->reserved[k] != 0) return WC_E_CORRUPT;
  return WC_OK;
}

inline Dict dict_of(const wc_header* h) {
  Dict d;
  for (int k = 0; k < 16; ++k) d.sym[k] = (k < h->n_dict && k < 15) ? h->dict[k] : 0;
  d.n_dict = h->n_dict;
  return d;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace wc
