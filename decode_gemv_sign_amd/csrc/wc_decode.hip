// wc_decode.hip — exact decode of a container into BF16 bit patterns.
//
// Page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%", section
// "Cómo funciona la compresión": the high byte (byte-split) or the 9-bit
// sign+exponent symbol (K15) is rebuilt from the dictionary, the code
// indices and the exact escape stream; the stored raw part is unchanged.
//
// HBM-bound: per weight it reads bpw/8 bytes of container and writes 2 bytes.
// Each wave owns a contiguous run of 2048-weight tiles, so the escape cursor
// is read once per wave (the escape index entry of its first tile) and then
// advanced by each tile's code-15 count.  Tiles stream through a per-wave
// LDS ring filled by global->LDS loads and are rebuilt in registers; tiles
// with escapes are patched (wc_tile.h), and every tile is stored with
// 16-byte non-temporal stores.
#include <type_traits>

#include "wc_launch.h"
#include "wc_tile.h"

namespace wc {

// Tiles per wave on tensors larger than one round of waves (measured on the
// layer set's 6144 x 24576 tensors, fraction of the 8 TB/s peak by tiles per
// wave 1 / 2 / 3 / 4 / 6: byte-split 0.76 / 0.70 / 0.70 / 0.69 / 0.67, K15
// 0.70 / 0.74 / 0.71 / 0.70 / 0.67).  Byte-split tiles carry almost no
// escapes, and a wave per tile spreads the loads widest; K15 tiles patch
// about 40 escapes each, whose record loads a two-tile run issues one tile
// ahead.
constexpr uint64_t kDecodeTilesBS = 1;
constexpr uint64_t kDecodeTilesK15 = 2;


struct DecodeArgs {
  const uint8_t* codes;
  const uint8_t* raw;
  const uint32_t* esc_pos;
  const uint8_t* esc_sym;
  const uint32_t* esc_idx;
  uint16_t* out;
  uint64_t n, n_esc, esc_last, raw_last, n_tiles, tiles_per_wave;
  uint64_t sym_last;  // last dword of the symbol stream's padded extent
  Dict dict;
};

// The ring has two slots per wave, one tile ahead of the one being rebuilt:
// 34 KB per 256-thread block, so four waves per SIMD fit.  (A third slot, two
// tiles ahead, costs the fourth wave; it measured the same on the large
// tensors and 11-13% slower on a 4096 x 4096 tensor, whose 4096 waves of two
// tiles fill one round only with four waves per SIMD.)
// CMP: the compact escape form (symbols only; every tile with escapes takes
// its symbols by rank from its run), a template argument so that the full
// form's kernel carries none of its branches.
// SLOTS: 2 for runs of several tiles; 1 when every wave takes one tile (the
// second slot would never be filled, and half the LDS lets twice the blocks
// share a compute unit).
template <int LAYOUT, bool CMP, int SLOTS>
__global__ __launch_bounds__(kBlockThreads) void k_decode(DecodeArgs a) {
  __shared__ uint32_t T2[256];
  // per wave: a ring of tile buffers filled by global->LDS loads, 4 KB per
  // slot (codes 1 KB + raw 2 KB + the first escape records); the whole slot
  // doubles as the escape stage of the tile just read from it
  constexpr int kWpb = kBlockThreads / kWave;
  __shared__ __attribute__((aligned(16))) uint32_t ring0[kWpb][kRingSlotDwords];
  __shared__ __attribute__((aligned(16))) uint32_t ring1[kWpb][SLOTS == 2 ? kRingSlotDwords : 4];
  build_pair_table<LAYOUT>(T2, a.dict);
  __syncthreads();

  const int lane = lane_id();
  const int wib = wave_in_block();
  const uint64_t wave = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + (uint64_t)wib;
  const uint64_t t0 = wave * a.tiles_per_wave;
  const uint64_t t1 = t0 + a.tiles_per_wave < a.n_tiles ? t0 + a.tiles_per_wave : a.n_tiles;
  if (t0 >= t1) return;

  // Every tile but the tensor's last is full.  Full tiles run in a software
  // pipeline: the next tiles' loads are in flight while tile t is rebuilt,
  // patched and stored.
  const uint64_t full_tiles = a.n / kTile;
  const uint64_t f1 = t1 < full_tiles ? t1 : full_tiles;  // end of this wave's full tiles
  uint64_t e = 0;  // escape cursor, read once the first tile's loads are in flight
  auto find_cursor = [&]() { e = escape_cursor(a.esc_idx, a.esc_pos, a.n_esc, a.n, t0 * kTile); };

  // Rebuild + escapes of tile t into out[16] (the lane's 4 groups); `stg` is
  // the tile's ring slot, free once the tile is in registers.  The tile's
  // first escape records come in `eb` (loaded while the previous tile was
  // processed).  As soon as this tile's escape count is known,
  // `issue_next(e_next)` issues the next tile's record loads; then a dense
  // tile's symbol run comes into `stg`, the last global->LDS loads issued.
  auto rebuild = [&](uint64_t t, const Lane4& l, const EscBatch& eb, auto&& issue_next,
                     uint32_t out[16], uint32_t* stg, bool ahead_ok) {
    uint32_t marks[kLaneGroups];
    const bool any = escape_marks(l, marks);
    const uint32_t cnt_wave = __ballot(any) ? wave_total(count_marks(marks)) : 0u;
    const bool dense = cnt_wave > (CMP ? 0u : kDenseMin);
    // compact form: a run that came with the tile serves it when it fits
    const bool ahead = ahead_ok && cnt_wave <= AheadSyms<LAYOUT>::value;
    issue_next(e + cnt_wave);
    const uint32_t off0 =
        dense && !ahead ? ring_load_symrun<LAYOUT>(a.esc_sym, a.sym_last, e, cnt_wave, stg) : 0u;
    rebuild_lane<LAYOUT>(T2, l, out);
    if (dense && ahead) {
      const uint32_t off = (uint32_t)((e * (LAYOUT == WC_LAYOUT_K15 ? 2u : 1u)) & 15u);
      // K15 tiles with few escapes per lane: by rank gather (wc_tile.h)
      uint32_t gm[kLaneGroups], gc[kLaneGroups], gf[kLaneGroups];
      bool few = false;
      if (LAYOUT == WC_LAYOUT_K15) {
        group_records(l, gm, gc, gf);
        few = !__ballot((gc[0] + gc[1] + gc[2] + gc[3]) > (uint32_t)kGatherMax);
      }
      if (few)
        patch_tile_gather<LAYOUT>(stg, out, gm, gf, lds_addr(stg + 768) + off);
      else
        patch_tile_symrun<LAYOUT>(l, out, stg + 768, off);
    } else if (dense) {
      wait_vm<0>();  // the symbol run is complete
      patch_tile_symrun<LAYOUT>(l, out, stg, off0);
    } else if (cnt_wave) {
      const uint64_t tile_start = t * kTile;
      const uint32_t tile_len = a.n - tile_start >= kTile ? kTile : (uint32_t)(a.n - tile_start);
      patch_tile<LAYOUT>(stg, out, group_mask(marks), a.esc_pos, a.esc_sym, a.n_esc, a.esc_last, e,
                         cnt_wave, tile_start, tile_len, eb);
    }
    e += cnt_wave;
  };

  if (t0 < f1) {
    // Full tiles stream through the LDS ring (wc_tile.h ring_*), one tile
    // ahead.  The loads need no registers, so the prefetch does not cost
    // occupancy.
    auto dma_tile = [&](uint64_t t, uint32_t* buf) {
      ring_load_tile<LAYOUT>(a.codes, a.raw, t * (kTile / kGroup), buf);
    };
    auto read_tile = [&](const uint32_t* buf, Lane4& l) { ring_read_tile<LAYOUT>(buf, l); };
    auto dma_eb = [&](uint64_t e0, uint32_t* buf) {
      if constexpr (CMP)
        ring_load_symrun_ahead<LAYOUT>(a.esc_sym, a.sym_last, a.n_esc, e0, buf);
      else
        ring_load_esc<LAYOUT>(a.esc_pos, a.esc_sym, (CMP ? 0ull : a.n_esc), a.esc_last, e0, buf);
    };
    auto read_eb = [&](const uint32_t* buf, uint64_t e0) {
      return ring_read_esc<LAYOUT>(buf, e0, (CMP ? 0ull : a.n_esc), a.esc_last);
    };
    uint32_t* const s0 = ring0[wib];
    uint32_t* const s1 = SLOTS == 2 ? ring1[wib] : ring0[wib];  // one slot: never refilled
    {
      // Two slots, one tile ahead.
      auto slot_buf = [&](auto slc) -> uint32_t* {
        return decltype(slc)::value % 2 == 0 ? s0 : s1;
      };
      dma_tile(t0, s0);  // in flight while the escape cursor is read
      find_cursor();
      dma_eb(e, s0);
      uint64_t t = t0;
      // Each step issues the next tile's ring loads, waits for the current
      // tile's ring and record loads (ring_wait_ahead; the last step, with no
      // next tile, waits for all), then stores the previous tile: deferred by
      // one step, the stores have a whole step to complete before a wait can
      // find them outstanding.
      uint32_t outA[16], outB[16];  // rebuilt tiles of even / odd steps
      auto store_tile = [&](uint64_t tt, const uint32_t out[16]) {
        u32x4* dst = (u32x4*)(a.out + tt * kTile) + lane;
#pragma unroll
        for (int k = 0; k < kLaneGroups; ++k)
          __builtin_nontemporal_store(u32x4{out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]},
                                      dst + kWave * k);
      };
      auto step = [&](auto slc, uint32_t* out, const uint32_t* prev) {
        constexpr int sl = decltype(slc)::value;
        wait_lgkm0();  // tile t-1's LDS reads and stage writes are done before it is refilled
        if (t + 1 < f1) {
          dma_tile(t + 1, slot_buf(std::integral_constant<int, sl + 1>{}));
          wait_vm<kRingAhead>();
        } else {
          wait_vm<0>();
        }
        if (t > t0) store_tile(t - 1, prev);
        Lane4 l;
        uint32_t* buf = slot_buf(slc);
        read_tile(buf, l);
        const EscBatch eb = read_eb(buf, e);
        uint32_t* nbuf = slot_buf(std::integral_constant<int, sl + 1>{});
        // (the next tile's records: with one slot there is never a next tile,
        // and the slot is this tile's escape stage, so nothing is loaded)
        rebuild(t, l, eb, [&](uint64_t en) { if (SLOTS == 2) dma_eb(en, nbuf); }, out, buf, CMP);
        ++t;
      };
      while (t + 2 <= f1) {
        step(std::integral_constant<int, 0>{}, outA, outB);
        step(std::integral_constant<int, 1>{}, outB, outA);
      }
      if (t < f1) {
        step(std::integral_constant<int, 0>{}, outA, outB);
        store_tile(t - 1, outA);
      } else {
        store_tile(t - 1, outB);
      }
      wait_vm<0>();  // the last step's (unused) record loads land before the stage is reused
      wait_lgkm0();
    }
  }
  if (t0 >= f1) find_cursor();  // a wave with only the partial last tile
  if (t1 > full_tiles) {
    // The tensor's partial last tile: groups past n are skipped, the group
    // that holds the last weight has its missing codes cleared (no phantom
    // escapes) and stores only its valid weights.
    const uint64_t tile_start = full_tiles * kTile;
    Lane4 l;
    uint32_t valid[kLaneGroups];
    const GroupBase gb = group_base(LAYOUT, a.codes, a.raw, full_tiles * (kTile / kGroup), a.raw_last);
#pragma unroll
    for (int k = 0; k < kLaneGroups; ++k) {
      const uint64_t w0 = tile_start + (uint64_t)(lane + kWave * k) * kGroup;
      valid[k] = w0 < a.n ? (a.n - w0 >= kGroup ? kGroup : (uint32_t)(a.n - w0)) : 0u;
      l.codes[k] = 0;
      l.raw[k][0] = l.raw[k][1] = 0;
      if (valid[k]) {
        load_group<LAYOUT>(gb, (uint32_t)(lane + kWave * k), l.codes[k], l.raw[k]);
        if (valid[k] < kGroup) l.codes[k] &= (1u << (4 * valid[k])) - 1u;
      }
    }
    uint32_t out[16];
    const EscBatch eb = load_esc<LAYOUT>(a.esc_pos, a.esc_sym, (CMP ? 0ull : a.n_esc), a.esc_last, e);
    // no global->LDS load is in flight here: ring0 is free
    rebuild(full_tiles, l, eb, [](uint64_t) {}, out, ring0[wib], false);
#pragma unroll
    for (int k = 0; k < kLaneGroups; ++k) {
      const uint64_t w0 = tile_start + (uint64_t)(lane + kWave * k) * kGroup;
      if (valid[k] == kGroup) {
        *(u32x4*)(a.out + w0) = u32x4{out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]};
      } else {
        for (uint32_t i = 0; i < valid[k]; ++i)
          a.out[w0 + i] = (uint16_t)(out[4 * k + (i >> 1)] >> (16u * (i & 1u)));
      }
    }
  }
}

// ---- raw layout: the weights stored as they are ---------------------------
// One 16-byte vector (8 weights) per thread and step, grid-stride.  Encode
// writes the container's header and pads its last vector with zeros (the
// stream's padding); decode writes only the n weights.

__global__ __launch_bounds__(kBlockThreads) void k_encode_raw(const uint16_t* __restrict__ w,
                                                              uint8_t* __restrict__ container,
                                                              uint64_t n, wc_header h) {
  if (blockIdx.x == 0 && threadIdx.x < WC_HEADER_BYTES / 4)
    ((uint32_t*)container)[threadIdx.x] = ((const uint32_t*)&h)[threadIdx.x];
  u32x4* dst = (u32x4*)(container + h.off_raw);
  const uint64_t nvec = (n + 7) / 8;
  for (uint64_t v = (uint64_t)blockIdx.x * kBlockThreads + threadIdx.x; v < nvec;
       v += (uint64_t)gridDim.x * kBlockThreads) {
    if (8 * v + 8 <= n) {
      dst[v] = __builtin_nontemporal_load((const u32x4*)w + v);
    } else {
      uint32_t d[4] = {0u, 0u, 0u, 0u};
      for (uint64_t i = 8 * v; i < n; ++i) d[(i & 7) >> 1] |= (uint32_t)w[i] << (16u * (uint32_t)(i & 1));
      dst[v] = u32x4{d[0], d[1], d[2], d[3]};
    }
  }
}

__global__ __launch_bounds__(kBlockThreads) void k_decode_raw(const uint8_t* __restrict__ raw,
                                                              uint16_t* __restrict__ out,
                                                              uint64_t n) {
  const u32x4* src = (const u32x4*)raw;
  const uint64_t nvec = (n + 7) / 8;
  for (uint64_t v = (uint64_t)blockIdx.x * kBlockThreads + threadIdx.x; v < nvec;
       v += (uint64_t)gridDim.x * kBlockThreads) {
    const u32x4 d = __builtin_nontemporal_load(src + v);
    if (8 * v + 8 <= n) {
      __builtin_nontemporal_store(d, (u32x4*)out + v);
    } else {
      for (uint64_t i = 8 * v; i < n; ++i) out[i] = (uint16_t)(d[(i & 7) >> 1] >> (16u * (uint32_t)(i & 1)));
    }
  }
}

static dim3 raw_grid(uint64_t n) {
  const uint64_t nvec = (n + 7) / 8;
  uint64_t blocks = (nvec + kBlockThreads - 1) / kBlockThreads;
  const uint64_t cap = (uint64_t)cu_count() * 16u;  // a few rounds' worth; the loop strides the rest
  blocks = blocks < cap ? blocks : cap;
  return dim3((unsigned)(blocks ? blocks : 1));
}

hipError_t launch_encode_raw(const wc_header& h, const uint16_t* w, uint8_t* container,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_encode_raw, raw_grid(h.n), dim3(kBlockThreads), 0, s, w, container, h.n, h);
  return hipGetLastError();
}

hipError_t launch_decode_raw(const wc_header& h, const uint8_t* container, uint16_t* out,
                             hipStream_t s) {
  if (h.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_decode_raw, raw_grid(h.n), dim3(kBlockThreads), 0, s, container + h.off_raw,
                     out, h.n);
  return hipGetLastError();
}

hipError_t launch_decode(const wc_header& h, const uint8_t* container, uint16_t* out,
                         hipStream_t s) {
  if (h.n == 0) return hipSuccess;
  if (h.layout == WC_LAYOUT_RAW) return launch_decode_raw(h, container, out, s);
  DecodeArgs a{};
  a.codes = container + h.off_codes;
  a.raw = container + h.off_raw;
  a.esc_pos = (const uint32_t*)(container + h.off_esc_pos);
  a.esc_sym = container + h.off_esc_sym;
  a.esc_idx = (const uint32_t*)(container + h.off_esc_idx);
  a.out = out;
  a.n = h.n;
  a.n_esc = h.n_esc;
  // with no escapes, the (never used) escape loads read the container header
  a.esc_last = h.n_esc ? h.n_esc - 1 : 0;
  a.sym_last = h.n_esc ? (h.off_esc_idx - h.off_esc_sym) / 4 - 1 : 0;
  if (h.n_esc == 0) {
    a.esc_pos = (const uint32_t*)container;
    a.esc_sym = container;
    a.esc_idx = (const uint32_t*)container;
  }
  const bool compact = (h.flags & WC_FLAG_COMPACT) != 0;
  if (compact) {
    // no positions: the (never used) position prefetch reads the header
    a.esc_last = 0;
    a.esc_pos = (const uint32_t*)container;
  }
  a.raw_last = pad16(raw_bytes(h.layout, h.n)) / 4 - 1;
  a.n_tiles = (h.n + kTile - 1) / kTile;
  // Short runs of tiles per wave keep the waves that run at the same time on
  // neighbouring memory (whole-tensor runs per resident wave measured 12%
  // slower than 4-tile runs, and shorter runs faster still, see above).  A
  // tensor that fits in one round of 3-tile runs of the waves the chip holds
  // at once (4 per SIMD, LDS-bound) takes runs that fill exactly one round.
  const uint64_t slots = (uint64_t)cu_count() * 4u * 4u;
  const bool one_round = a.n_tiles <= 3 * slots;
  a.tiles_per_wave = one_round ? (a.n_tiles + slots - 1) / slots
                               : (h.layout == WC_LAYOUT_K15 ? kDecodeTilesK15 : kDecodeTilesBS);
  const uint64_t waves = (a.n_tiles + a.tiles_per_wave - 1) / a.tiles_per_wave;
  const uint64_t wpb = kBlockThreads / kWave;
  const dim3 grid((unsigned)((waves + wpb - 1) / wpb));
  a.dict = dict_of(&h);
  const dim3 blk(kBlockThreads);
  const bool one = a.tiles_per_wave == 1;
  if (h.layout == WC_LAYOUT_K15) {
    if (compact) {
      if (one) hipLaunchKernelGGL((k_decode<WC_LAYOUT_K15, true, 1>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((k_decode<WC_LAYOUT_K15, true, 2>), grid, blk, 0, s, a);
    } else {
      if (one) hipLaunchKernelGGL((k_decode<WC_LAYOUT_K15, false, 1>), grid, blk, 0, s, a);
      else hipLaunchKernelGGL((k_decode<WC_LAYOUT_K15, false, 2>), grid, blk, 0, s, a);
    }
  } else if (compact) {
    if (one) hipLaunchKernelGGL((k_decode<WC_LAYOUT_BYTESPLIT, true, 1>), grid, blk, 0, s, a);
    else hipLaunchKernelGGL((k_decode<WC_LAYOUT_BYTESPLIT, true, 2>), grid, blk, 0, s, a);
  } else {
    if (one) hipLaunchKernelGGL((k_decode<WC_LAYOUT_BYTESPLIT, false, 1>), grid, blk, 0, s, a);
    else hipLaunchKernelGGL((k_decode<WC_LAYOUT_BYTESPLIT, false, 2>), grid, blk, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace wc
