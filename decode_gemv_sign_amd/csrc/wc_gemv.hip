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
// y[b][r] = sum_c W[r][c] x[b][c].  A wave walks 2048-weight tiles along
// its rows: each lane rebuilds its 4 groups of 8 weights (wc_tile.h),
// multiplies them with the matching x values by v_dot2_f32_bf16 (exact BF16
// products, fp32 accumulate), and at the row's end the 64 lane partials are
// summed by butterfly shuffles.  HBM-bound at batch 1 and 4: per weight bpw/8
// bytes of container are read (x stays in L2).  Rows made of whole tiles at
// batch <= 4 stream through an LDS ring (k_decode_gemv_ring); other shapes
// use a register ring (k_decode_gemv); batches of 8 and more go to the
// matrix-core kernel (wc_gemm.hip) when the shape fits it.
//
// Rows whose length is not a multiple of 8 (a group would straddle two rows)
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
  const uint32_t* esc_idx;
  const uint16_t* w;  // plain BF16 weights (comparator)
  const uint16_t* x;
  float* y;
  uint64_t rows, cols, n_esc, esc_last, raw_last, rows_per_wave;
  uint64_t sym_last;  // last dword of the symbol stream's padded extent
  uint32_t compact;    // escape symbols only (no position stream)
  uint32_t batch;
  uint32_t wpr;        // ring kernel, split rows: parts per row (rows, cols are the parts')
  uint64_t x_cols;     // ring kernel, split rows: length of an x row (the real cols)
  Dict dict;
};

// acc += the lane's 16 weight pairs (4 groups) times x[g*8 .. g*8+8) of its
// groups, for batch row b of x (x row length `cols`).
__device__ inline float dot_lane(const uint32_t w[16], const uint32_t xv[16], float acc) {
  float s0 = acc, s1 = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; k += 2) {
    s0 = dot2(w[k], xv[k], s0);
    s1 = dot2(w[k + 1], xv[k + 1], s1);
  }
  return s0 + s1;
}

// x values of the lane's 4 groups; `xt` points at the tile's first x value.
__device__ inline void load_x_lane(const uint16_t* __restrict__ xt, const uint32_t lg[4],
                                   uint32_t xv[16]) {
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    const u32x4 v = *((const u32x4*)xt + lg[k]);
    xv[4 * k] = v[0]; xv[4 * k + 1] = v[1]; xv[4 * k + 2] = v[2]; xv[4 * k + 3] = v[3];
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

#ifndef WC_GEMV_DEPTH
#define WC_GEMV_DEPTH 2
#endif
#ifndef WC_GEMV_PREFETCH_X
#define WC_GEMV_PREFETCH_X 1
#endif
#ifndef WC_GATHER
#define WC_GATHER 1
#endif
// K15 tiles with few escapes per lane are patched by rank gather at batch 1
// (measured on 6144 x 24576 N(0, 0.015), compact form: 80 -> 67 us); the
// window path stays faster for byte-split, whose windows are cheap
constexpr bool kGatherOn = WC_GATHER;
constexpr int kGemvDepth = WC_GEMV_DEPTH;            // tiles in the prefetch ring
constexpr bool kGemvPrefetchX = WC_GEMV_PREFETCH_X;  // x rides in the ring at batch 1

// Position (row, tile-in-row) in a wave's tile sequence.
struct TileCursor {
  uint64_t r, ct;
  __device__ void next(uint64_t tpr) {
    if (++ct == tpr) {
      ct = 0;
      ++r;
    }
  }
};

// Software pipeline over nq tiles with a ring of D register slots: tile q+D-1
// is loaded just before tile q is processed.  init(slot 0) runs once the
// first tiles' loads are issued (it may wait on memory of its own).  The
// ring is unrolled, so every slot index is static (no register copies,
// which would wait on the loads),
// and loads past the end re-read the last tile (their data is unused), so the
// loads in flight are the same on every path.  process(cursor, slot, next)
// may also fill fields of the next tile's slot that the load does not touch
// (the next tile's first escape records).
template <int D, typename Slot, typename Init, typename Load, typename Process>
__device__ inline void run_ring(uint64_t nq, TileCursor start, uint64_t tpr, Init&& init,
                                Load&& load, Process&& process) {
  Slot s[D];
  TileCursor lc = start, pc = start;
  uint64_t lq = 0;  // index of the tile lc points at
  auto load_next = [&](Slot& slot) {
    load(lc, slot);
    if (lq + 1 < nq) {
      lc.next(tpr);
      ++lq;
    }
  };
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load_next(s[i]);
  init(s[0]);  // after the first loads are in flight
  for (uint64_t q = 0; q < nq; q += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      load_next(s[(i + D - 1) % D]);
      if (q + i >= nq) return;
      process(pc, s[i], s[(i + 1) % D]);
      pc.next(tpr);
    }
  }
}

// Row tile (r, ct) = groups [256 ct, 256 ct + 256) of row r; lane L takes
// tile groups lg_k = L + 64 k that are inside the row (a lane past the row end
// reloads the row's last group and drops it, so every path issues the same
// loads).  Only a row's last tile can be partial (a wave-uniform test).
struct RowTile {
  uint32_t lg[kLaneGroups];  // tile-local group per k (clamped)
  uint32_t act;              // bit k: group k is inside the row
  bool partial;              // some lane's group lies past the row end
};

__device__ inline RowTile row_tile(uint64_t ct, uint64_t gpr) {
  RowTile t;
  const uint64_t left = gpr - ct * (kTile / kGroup);  // groups of the row from this tile on
  t.partial = left < (uint64_t)(kTile / kGroup);
  t.act = 0;
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) {
    const uint32_t g = (uint32_t)(lane_id() + kWave * k);
    const bool in = !t.partial || g < left;
    t.lg[k] = in ? g : (uint32_t)left - 1u;
    t.act |= (in ? 1u : 0u) << k;
  }
  return t;
}

// One wave per run of `rows_per_wave` consecutive rows.  Its tiles form one
// sequence over those rows; the loads of tile q+1 (coded weights, and x at
// batch 1) are in flight while tile q is rebuilt, patched and multiplied, two
// register sets alternating (the loop is unrolled by two), and the escape
// cursor found for the run's first row is carried to its end.
// CMP: the compact escape form (symbols only), a template argument so that
// the full form's kernels carry none of its branches.
template <int LAYOUT, int B, bool CMP>
__global__ __launch_bounds__(kBlockThreads) void k_decode_gemv(GemvArgs a) {
  __shared__ uint32_t T2[256];
  __shared__ __attribute__((aligned(16))) uint32_t stage[kBlockThreads / kWave][kStageDwords];
  build_pair_table<LAYOUT>(T2, a.dict);
  __syncthreads();

  const int wib = wave_in_block();
  const uint64_t wave = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + (uint64_t)wib;
  const uint64_t r0 = wave * a.rows_per_wave;
  if (r0 >= a.rows) return;
  const uint64_t r1 = r0 + a.rows_per_wave < a.rows ? r0 + a.rows_per_wave : a.rows;
  const uint64_t gpr = a.cols / kGroup;                              // groups per row
  const uint64_t tpr = (gpr + kTile / kGroup - 1) / (kTile / kGroup);  // tiles per row

  // x at batch 1 rides along with the weights in the prefetch ring when
  // kGemvPrefetchX; otherwise it is read (from L2) when the tile is used.
  constexpr bool kXpf = B == 1 && kGemvPrefetchX;
  struct Slot {
    Lane4 l;
    uint32_t xv[kXpf ? 16 : 1];
    uint32_t act;
    EscBatch eb;  // the tile's first escape records
  };
  auto load_tile = [&](const TileCursor& c, Slot& s) {
    const RowTile rt = row_tile(c.ct, gpr);
    s.act = rt.act;
    const GroupBase gb =
        group_base(LAYOUT, a.codes, a.raw, c.r * gpr + c.ct * (kTile / kGroup), a.raw_last);
#pragma unroll
    for (int k = 0; k < kLaneGroups; ++k) {
      load_group<LAYOUT>(gb, rt.lg[k], s.l.codes[k], s.l.raw[k]);
      if (rt.partial && !((rt.act >> k) & 1u)) s.l.codes[k] = 0;  // no weights, no escapes
    }
    if (kXpf) load_x_lane(a.x + c.ct * kTile, rt.lg, s.xv);
  };

  uint64_t e = 0;  // escape cursor: found in init, while the first tile loads
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;

  auto process = [&](const TileCursor& c, const Slot& s, Slot& sn) {
    const RowTile rt = row_tile(c.ct, gpr);
    uint32_t xv[kXpf ? 1 : 16];
    if (!kXpf && B == 1) load_x_lane(a.x + c.ct * kTile, rt.lg, xv);  // in flight during the rebuild
    uint32_t marks[kLaneGroups];
    const bool any = escape_marks(s.l, marks);
    const uint32_t cnt_wave = __ballot(any) ? wave_total(count_marks(marks)) : 0u;
    // the next tile's first records, in flight while this tile is rebuilt
    sn.eb = load_esc<LAYOUT>(a.esc_pos, a.esc_sym, (CMP ? 0ull : a.n_esc), a.esc_last, e + cnt_wave);
    uint32_t w[16];
    rebuild_lane<LAYOUT>(T2, s.l, w);
    if (cnt_wave > (CMP ? 0u : kDenseMin)) {
      patch_tile_windows<LAYOUT>(s.l, w, a.esc_sym, a.sym_last, e);
    } else if (cnt_wave) {
      const uint64_t tile_start = c.r * a.cols + c.ct * kTile;
      const uint64_t left = a.cols - c.ct * kTile;
      patch_tile<LAYOUT>(stage[wib], w, group_mask(marks), a.esc_pos, a.esc_sym, a.n_esc, a.esc_last, e,
                         cnt_wave, tile_start, left >= kTile ? kTile : (uint32_t)left, s.eb);
    }
    e += cnt_wave;
    // groups outside the row contribute nothing
    if (rt.partial) {
#pragma unroll
      for (int k = 0; k < kLaneGroups; ++k)
        if (!((s.act >> k) & 1u)) w[4 * k] = w[4 * k + 1] = w[4 * k + 2] = w[4 * k + 3] = 0;
    }
    if (B == 1) {
      if constexpr (kXpf)
        acc[0] = dot_lane(w, s.xv, acc[0]);
      else
        acc[0] = dot_lane(w, xv, acc[0]);
    } else {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        uint32_t xb[16];
        load_x_lane(a.x + (uint64_t)b * a.cols + c.ct * kTile, rt.lg, xb);
        acc[b] = dot_lane(w, xb, acc[b]);
      }
    }
    if (c.ct + 1 == tpr) {
      store_row<B>(acc, a.y, a.rows, c.r);
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    }
  };

  auto init = [&](Slot& s0) {
    e = escape_cursor_at(CMP, a.esc_idx, a.esc_pos, a.codes, a.n_esc, a.rows * a.cols,
                         r0 * a.cols);
    s0.eb = load_esc<LAYOUT>(a.esc_pos, a.esc_sym, (CMP ? 0ull : a.n_esc), a.esc_last, e);
  };
  run_ring<kGemvDepth, Slot>((r1 - r0) * tpr, TileCursor{r0, 0}, tpr, init, load_tile, process);
}

// k_decode_gemv for rows of whole tiles (cols a multiple of 2048): the coded
// tiles and their first escape records stream through a two-slot LDS ring
// filled by global->LDS loads (wc_tile.h ring_*), one tile ahead, instead
// of the register ring.  At batch 1, x for the next tile rides in
// registers; larger batches read x when the tile is used.  Each step issues
// the next tile's loads first and waits for them before its dot product.
//
// SPLIT: a row of W[R][C] is split into a.wpr parts of whole tiles, each a
// row of the same bytes viewed as W[R * wpr][C / wpr] (row-major order and
// tile numbering are unchanged, so the escape index serves as it is).  The
// kernel runs on that view, one part per wave (a.rows, a.cols are the
// parts'; a.rows_per_wave is 1); part p of a row reads x from column
// p * a.cols on, and the waves of the block that hold one row's parts add
// their sums in LDS in column order, so the result does not depend on which
// wave ends first.  Measured at batch 4 on 6144 x 24576 (4 parts of 3
// tiles): 82 against 87 us byte-split, 89 against 91 K15; 2 parts of 6 are
// faster still (the launcher's numbers).  At batch 1 it was slower (57
// against 50 with 4 parts); with 2 parts it pays only for K15 on tensors
// with dense escape rows (the launcher's rule).
template <int LAYOUT, int B, bool CMP, bool SPLIT, uint32_t SLOT = kRingSlotDwords,
          int WPB = kBlockThreads / kWave>
__global__ __launch_bounds__(kWave * WPB) void k_decode_gemv_ring(GemvArgs a) {
  // 16-byte chunks of symbol run a slot takes ahead (wc_tile.h run_ahead)
  constexpr uint32_t kAheadChunks = (4 * SLOT - 3104) / 16;
  static_assert(kAheadChunks >= 66 && kAheadChunks <= 128, "slot sizes of the ring");
  // symbols such a run holds (the rest of a longer run is loaded once the
  // tile is in registers)
  constexpr uint32_t kAheadCap = run_ahead_syms(kAheadChunks, LAYOUT);
  __shared__ uint32_t T2[256];
  __shared__ __attribute__((aligned(16))) uint32_t ring0[WPB][SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t ring1[WPB][SLOT];
  __shared__ float part_sum[WPB][SPLIT ? B : 1];

  const int lane = lane_id();
  const int wib = wave_in_block();
  // SPLIT in 8-wave blocks: the block holds 8 / wpr whole rows, part-major
  // (waves 0 .. rpb - 1 take part 0 of consecutive rows, and so on), so the
  // waves of one part read the same x columns.  4-wave blocks keep a row's
  // parts on neighbouring waves (rpb = 1), measured 2% faster there (K15,
  // banded 6144 x 24576, batch 4).
  constexpr bool kPartMajor = SPLIT && WPB == 8;
  const uint32_t rpb = kPartMajor ? (uint32_t)WPB / a.wpr : 1u;
  const uint64_t r0 = kPartMajor ? ((uint64_t)blockIdx.x * rpb + (uint32_t)wib % rpb) * a.wpr + (uint32_t)wib / rpb
                                 : ((uint64_t)blockIdx.x * WPB + (uint64_t)wib) * a.rows_per_wave;
  // Every thread of the block builds its share of the pair table and
  // reaches the barrier after it (waves without rows, in the else branch);
  // waves with rows issue their first loads before that.
  if (r0 < a.rows) {
  const uint64_t r1 = r0 + a.rows_per_wave < a.rows ? r0 + a.rows_per_wave : a.rows;
  const uint64_t gpr = a.cols / kGroup;
  const uint64_t tpr = a.cols / kTile;  // whole tiles
  const uint64_t nq = (r1 - r0) * tpr;
  uint32_t* const s0 = ring0[wib];
  uint32_t* const s1 = ring1[wib];

  constexpr bool kXpf = B == 1;
  // K15 symbol windows per LDS round trip: one at batch 4, where the
  // batch's accumulators leave no registers for two
  constexpr int kSymPass = B == 1 ? 2 : 1;
  uint32_t lg[kLaneGroups];
#pragma unroll
  for (int k = 0; k < kLaneGroups; ++k) lg[k] = (uint32_t)lane + kWave * k;
  // tile q of the wave: row r0 + q / tpr, tile q % tpr of the row (loaded
  // for q < nq only)
  TileCursor lc{r0, 0};
  // x of a row's part p starts at column p * a.cols
  auto xrow = [&](uint64_t r) -> const uint16_t* {
    return SPLIT ? a.x + (r % a.wpr) * a.cols : a.x;
  };
  auto load_next = [&](uint32_t* buf, uint32_t xv[16]) {
    ring_load_tile<LAYOUT>(a.codes, a.raw, lc.r * gpr + lc.ct * (kTile / kGroup), buf);
    if (kXpf) load_x_lane(xrow(lc.r) + lc.ct * kTile, lg, xv);
    lc.next(tpr);
  };

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  // Escape cursors from the escape index: rows are whole tiles, so the
  // wave's tile q is tile r0 * tpr + q of the tensor and its first record is
  // that tile's index entry.  Lane i holds the entry of tile qb + i (64 at a
  // time, clamped to n_esc), so the records of the next tile can be loaded
  // before this tile's escapes are counted.
  const uint64_t last_entry = a.rows * tpr;  // the closing entry
  uint64_t qb = 0;
  uint32_t iv = 0;
  auto load_iv = [&]() {
    if (a.n_esc) {
      uint64_t j = r0 * tpr + qb + (uint64_t)lane;
      j = j < last_entry ? j : last_entry;
      const uint32_t v = a.esc_idx[j];
      iv = v < a.n_esc ? v : (uint32_t)a.n_esc;
    }
  };
  // Entries of tiles q .. q + 2 in the lanes (a tile's first record, and its
  // escape count as the next tile's first record minus its own); called
  // with q non-decreasing.
  auto window = [&](uint64_t q) {
    if (q + 2 - qb >= (uint64_t)kWave) {
      qb = q;
      load_iv();
    }
  };
  auto entry = [&](uint64_t q) -> uint64_t {
    return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)iv, (int)(q - qb));
  };

  uint32_t x0[kXpf ? 16 : 1], x1[kXpf ? 16 : 1];
  load_next(s0, x0);  // in flight while the escape index is read
  load_iv();
  build_pair_table<LAYOUT, true>(T2, a.dict);  // while those loads are in flight
  __syncthreads();
  // With a tile's ring loads go its first records, or the start of its
  // symbol run, as much of it as the index says the tile holds (the same
  // number of loads either way): always in the compact form, which has no
  // records, and in the byte-split full form for tiles that the index shows
  // dense and whose run the slot holds whole (a dense tile is patched from
  // its run, so its records are of no use).  Measured at batch 4: 14336 x
  // 4096, 37.7 -> 35.7 us; 4096 x 14336, 37.2 -> 33.0.  K15 full-form tiles
  // measured slower that way (4096 x 4096, batch 1: 10.1 -> 12.7 us).
  constexpr bool kFullAhead = LAYOUT == WC_LAYOUT_BYTESPLIT;
  auto run_taken = [&](uint64_t cnt) -> bool {
    return CMP || (kFullAhead && cnt > kDenseMin && cnt <= kAheadCap);
  };
  auto load_records = [&](uint64_t e0, uint64_t cnt, uint32_t* buf) {
    if (run_taken(cnt))
      ring_load_run_ahead<LAYOUT>(a.esc_sym, a.sym_last, a.n_esc, e0, cnt, kAheadChunks, buf);
    else
      ring_load_esc<LAYOUT>(a.esc_pos, a.esc_sym, (CMP ? 0ull : a.n_esc), a.esc_last, e0, buf);
  };
  window(0);
  load_records(entry(0), entry(1) - entry(0), s0);
  TileCursor pc{r0, 0};

  auto step = [&](uint64_t q, uint32_t* buf, uint32_t* nbuf, uint32_t xv[16], uint32_t xn[16]) {
    wait_lgkm0();  // the previous tile's LDS reads and stage writes are done
    window(q);
    const uint64_t e = entry(q);
    // The next tile's ring loads and its first records (or run) go out
    // together.  The first tile's ring and record loads are complete once at
    // most those 3 + 2 loads are outstanding, or none when there is no next
    // tile; later tiles' loads were issued before the previous tile's full
    // wait.
    if (q + 1 < nq) {
      load_next(nbuf, xn);
      const uint64_t e1 = entry(q + 1);
      load_records(e1, entry(q + 2) - e1, nbuf);
      if (q == 0) wait_vm<kRingAheadEsc>();
    } else if (q == 0) {
      wait_vm<0>();
    }
    Lane4 l;
    ring_read_tile<LAYOUT>(buf, l);
    const EscBatch eb = ring_read_esc<LAYOUT>(buf, e, (CMP ? 0ull : a.n_esc), a.esc_last);
    uint32_t xb1[kXpf ? 1 : 16];
    if (!kXpf && B == 1) load_x_lane(a.x + pc.ct * kTile, lg, xb1);
    // Batches 2..4: x of the first XE batch rows issued now, in flight during
    // the rebuild and patch (both rows at batch 2, one above, where more
    // registers cost waves).  6144 x 24576 banded: batch 2 66.6 -> 64.3 us
    // byte-split, 68.9 -> 67.6 K15; batch 4 K15 86.1 -> 84.3.
    constexpr int XE = B == 2 ? 2 : (B > 2 ? 1 : 0);
    uint32_t xe[XE > 0 ? XE : 1][16];
#pragma unroll
    for (int b = 0; b < XE; ++b)
      load_x_lane(xrow(pc.r) + (uint64_t)b * (SPLIT ? a.x_cols : a.cols) + pc.ct * kTile, lg, xe[b]);
    uint32_t marks[kLaneGroups];
    const bool any = escape_marks(l, marks);
    const uint32_t cnt_wave = __ballot(any) ? wave_total(count_marks(marks)) : 0u;
    // A tile whose run came with it is patched from there when the run
    // holds all its escapes (always, unless the container's index and codes
    // disagree); other dense tiles load their run into the slot now (free:
    // the tile is in registers); sparse ones use their records.
    const bool taken = run_taken(entry(q + 1) - e);
    const bool dense = cnt_wave > (CMP ? 0u : kDenseMin);
    const bool ahead = taken && cnt_wave <= kAheadCap;
    const bool by_run = cnt_wave && (ahead || dense);  // patched from a symbol run
    const uint32_t off0 =
        by_run && !ahead ? ring_load_symrun<LAYOUT>(a.esc_sym, a.sym_last, e, cnt_wave, buf) : 0u;
    uint32_t w[16];
    rebuild_lane<LAYOUT>(T2, l, w);
    if (by_run) {
      // the run that came with the tile (from dword 768), or the one just
      // loaded (from dword 0)
      uint32_t* run = buf;
      uint32_t off = off0;
      if (ahead) {
        run = buf + 768;
        off = (uint32_t)((e * (LAYOUT == WC_LAYOUT_K15 ? 2u : 1u)) & 15u);
      } else {
        wait_vm<0>();
      }
      uint32_t gm[kLaneGroups], gc[kLaneGroups], gf[kLaneGroups];
      bool few = false;
      if (kGatherOn && B == 1 && LAYOUT == WC_LAYOUT_K15 && ahead) {
        group_records(l, gm, gc, gf);
        few = !__ballot((gc[0] + gc[1] + gc[2] + gc[3]) > (uint32_t)kGatherMax);
      }
      if (few)
        patch_tile_gather<LAYOUT>(buf, w, gm, gf, lds_addr(run) + off);
      else
        patch_tile_symrun<LAYOUT, kSymPass>(l, w, run, off);
    } else if (cnt_wave) {
      patch_tile<LAYOUT>(buf, w, group_mask(marks), a.esc_pos, a.esc_sym, a.n_esc, a.esc_last, e,
                         cnt_wave, pc.r * a.cols + pc.ct * kTile, kTile, eb);
    }
    // Full wait: x is read by ordinary loads, which the compiler awaits with
    // vmcnt(0) anyway while global->LDS loads are pending; it also completes
    // the next tile's ring and record loads.
    wait_vm<0>();
    if (B == 1) {
      acc[0] = dot_lane(w, kXpf ? xv : xb1, acc[0]);
    } else {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (b < XE) {
          acc[b] = dot_lane(w, xe[b < XE ? b : 0], acc[b]);
        } else {
          uint32_t xb[16];
          load_x_lane(xrow(pc.r) + (uint64_t)b * (SPLIT ? a.x_cols : a.cols) + pc.ct * kTile, lg, xb);
          acc[b] = dot_lane(w, xb, acc[b]);
        }
      }
    }
    if (pc.ct + 1 == tpr) {
      if constexpr (SPLIT) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float t = wave_sum_f32(acc[b]);
          if (lane == 0) part_sum[wib][b] = t;
        }
      } else {
        store_row<B>(acc, a.y, a.rows, pc.r);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    }
    pc.next(tpr);
  };
  uint64_t q = 0;
  for (; q + 1 < nq; q += 2) {
    step(q, s0, s1, x0, x1);
    step(q + 1, s1, s0, x1, x0);
  }
  if (q < nq) step(q, s0, s1, x0, x1);
  wait_vm<0>();  // the last tile's (unused) record loads land before the wave ends
  } else {
    build_pair_table<LAYOUT, true>(T2, a.dict);
    __syncthreads();
  }
  if constexpr (SPLIT) {
    __syncthreads();
    if (r0 < a.rows && r0 % a.wpr == 0 && lane == 0) {
      const uint64_t rows_real = a.rows / a.wpr;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float t = part_sum[wib][b];
        for (uint32_t k = 1; k < a.wpr; ++k) t += part_sum[wib + k * rpb][b];
        a.y[(uint64_t)b * rows_real + r0 / a.wpr] = t;
      }
    }
  }
}

// The same wave/tile schedule as k_decode_gemv with W read as plain BF16
// (16 bytes per group) and no rebuild: the comparison kernel.
template <int B>
__global__ __launch_bounds__(kBlockThreads) void k_gemv_bf16(GemvArgs a) {
  const uint64_t wave = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + (uint64_t)wave_in_block();
  const uint64_t r0 = wave * a.rows_per_wave;
  if (r0 >= a.rows) return;
  const uint64_t r1 = r0 + a.rows_per_wave < a.rows ? r0 + a.rows_per_wave : a.rows;
  const uint64_t gpr = a.cols / kGroup;
  const uint64_t tpr = (gpr + kTile / kGroup - 1) / (kTile / kGroup);

  constexpr bool kXpf = B == 1 && kGemvPrefetchX;
  struct Slot {
    uint32_t w[16];
    uint32_t xv[kXpf ? 16 : 1];
    uint32_t act;
  };
  auto load_tile = [&](const TileCursor& c, Slot& s) {
    const RowTile rt = row_tile(c.ct, gpr);
    s.act = rt.act;
    const u32x4* wr = (const u32x4*)(a.w + c.r * a.cols + c.ct * kTile);
#pragma unroll
    for (int k = 0; k < kLaneGroups; ++k) {
      const u32x4 v = __builtin_nontemporal_load(wr + rt.lg[k]);
      s.w[4 * k] = v[0]; s.w[4 * k + 1] = v[1]; s.w[4 * k + 2] = v[2]; s.w[4 * k + 3] = v[3];
    }
    if (kXpf) load_x_lane(a.x + c.ct * kTile, rt.lg, s.xv);
  };
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  auto process = [&](const TileCursor& c, const Slot& s, Slot&) {
    const RowTile rt = row_tile(c.ct, gpr);
    uint32_t xv[kXpf ? 1 : 16];
    if (!kXpf && B == 1) load_x_lane(a.x + c.ct * kTile, rt.lg, xv);
    uint32_t w[16];
#pragma unroll
    for (int k = 0; k < kLaneGroups; ++k) {
      const bool in = !rt.partial || ((s.act >> k) & 1u);
#pragma unroll
      for (int j = 0; j < 4; ++j) w[4 * k + j] = in ? s.w[4 * k + j] : 0u;
    }
    if (B == 1) {
      if constexpr (kXpf)
        acc[0] = dot_lane(w, s.xv, acc[0]);
      else
        acc[0] = dot_lane(w, xv, acc[0]);
    } else {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        uint32_t xb[16];
        load_x_lane(a.x + (uint64_t)b * a.cols + c.ct * kTile, rt.lg, xb);
        acc[b] = dot_lane(w, xb, acc[b]);
      }
    }
    if (c.ct + 1 == tpr) {
      store_row<B>(acc, a.y, a.rows, c.r);
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = 0.0f;
    }
  };
  run_ring<kGemvDepth, Slot>((r1 - r0) * tpr, TileCursor{r0, 0}, tpr, [](Slot&) {}, load_tile,
                             process);
}

// ---- generic shapes (cols % 8 != 0): one weight per lane per step ---------
// The launchers hand these kernels at most 16 input rows at a time.
constexpr int kGenericBatch = 16;

__device__ inline float bf16f(uint32_t b) { return __uint_as_float(b << 16); }

template <int LAYOUT>
__global__ __launch_bounds__(kBlockThreads) void k_decode_gemv_generic(GemvArgs a) {
  __shared__ uint16_t dsym[16];
  if (threadIdx.x < 16) dsym[threadIdx.x] = a.dict.sym[threadIdx.x];
  __syncthreads();
  const int lane = lane_id();
  const uint64_t r = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + (uint64_t)wave_in_block();
  if (r >= a.rows) return;
  const uint64_t row_start = r * a.cols;
  const uint64_t n = a.rows * a.cols;
  const uint64_t raw_len = raw_bytes(LAYOUT, n);
  uint64_t e = escape_cursor_at(a.compact, a.esc_idx, a.esc_pos, a.codes, a.n_esc, n, row_start);
  float acc[kGenericBatch];
#pragma unroll
  for (int b = 0; b < kGenericBatch; ++b) acc[b] = 0.0f;
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
      for (int b = 0; b < kGenericBatch; ++b)
        if (b < (int)a.batch) acc[b] = fmaf(wf, bf16f(a.x[(uint64_t)b * a.cols + c]), acc[b]);
    }
    e += (uint64_t)__popcll(m);
  }
#pragma unroll
  for (int b = 0; b < kGenericBatch; ++b) {
    if (b < (int)a.batch) {
      const float s = wave_sum_f32(acc[b]);
      if (lane == 0) a.y[(uint64_t)b * a.rows + r] = s;
    }
  }
}

__global__ __launch_bounds__(kBlockThreads) void k_gemv_bf16_generic(GemvArgs a) {
  const int lane = lane_id();
  const uint64_t r = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + (uint64_t)wave_in_block();
  if (r >= a.rows) return;
  float acc[kGenericBatch];
#pragma unroll
  for (int b = 0; b < kGenericBatch; ++b) acc[b] = 0.0f;
  for (uint64_t c = (uint64_t)lane; c < a.cols; c += kWave) {
    const float wf = bf16f(a.w[r * a.cols + c]);
#pragma unroll
    for (int b = 0; b < kGenericBatch; ++b)
      if (b < (int)a.batch) acc[b] = fmaf(wf, bf16f(a.x[(uint64_t)b * a.cols + c]), acc[b]);
  }
#pragma unroll
  for (int b = 0; b < kGenericBatch; ++b) {
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

// Batches from this size on take the matrix-core kernels of wc_gemm.hip
// (when cols is a multiple of 32): the fused kernel from 5, where the 1D
// kernels need two passes over W (6144 x 24576 banded, batch 5: 133 -> 94
// us byte-split, 144 -> 126 K15; at batch 4 the LDS ring is faster there,
// 84 against 92), the plain one from 4 (86 -> 84 us; 4096 x 4096 13.0 ->
// 9.8).  Unused lanes of the 16-wide batch operand re-read x row 0.
#ifndef WC_MFMA_MIN_BATCH
#define WC_MFMA_MIN_BATCH 5
#endif
#ifndef WC_MFMA_MIN_BATCH_PLAIN
#define WC_MFMA_MIN_BATCH_PLAIN 4
#endif
constexpr uint32_t kMfmaMinBatch = WC_MFMA_MIN_BATCH;
constexpr uint32_t kMfmaMinBatchPlain = WC_MFMA_MIN_BATCH_PLAIN;
// Rows of whole tiles take the LDS-ring kernel.
#ifndef WC_GEMV_RING
#define WC_GEMV_RING 1
#endif
constexpr bool kGemvRing = WC_GEMV_RING;
#ifndef WC_SPLIT_MIN_TILES
#define WC_SPLIT_MIN_TILES 4
#endif
constexpr uint64_t kSplitMinTiles = WC_SPLIT_MIN_TILES;  // rows of more tiles are split at batches 3 and 4

static dim3 row_grid(uint64_t rows) {
  const uint64_t wpb = kBlockThreads / kWave;
  return dim3((unsigned)((rows + wpb - 1) / wpb));
}

// Rows per wave: enough tiles per wave (about 4) to amortise each wave's
// start (escape cursor, first loads), while leaving many waves for the
// scheduler to balance.
#ifndef WC_GEMV_MIN_TILES
#define WC_GEMV_MIN_TILES 4
#endif
static uint64_t rows_per_wave(uint64_t rows, uint64_t cols) {
  const uint64_t tpr = (cols + kTile - 1) / kTile;
  const uint64_t rpw = tpr >= WC_GEMV_MIN_TILES ? 1 : (WC_GEMV_MIN_TILES + tpr - 1) / tpr;
  // Less than one round of waves (4 per SIMD): spread the rows over one
  // round instead, as few per wave as fill it.
  const uint64_t slots = (uint64_t)cu_count() * 16u;
  if ((rows + rpw - 1) / rpw < slots) return rows > slots ? (rows + slots - 1) / slots : 1;
  return rpw;
}

static dim3 wave_grid(uint64_t rows, uint64_t rpw) {
  const uint64_t waves = (rows + rpw - 1) / rpw;
  const uint64_t wpb = kBlockThreads / kWave;
  return dim3((unsigned)((waves + wpb - 1) / wpb));
}

// LDS ring slots of k_decode_gemv_ring.  A 4160-byte slot (4 KB of tile and
// records, room for a 1056-byte symbol run ahead) lets 4 blocks share a
// compute unit.  Byte-split at batch 1 on grids of more than one round of
// such waves, with 8 or more tiles per wave, takes 5152-byte slots instead (3
// blocks per compute unit): their 2048-byte run ahead holds a tile's symbols
// even when nearly every weight escapes, so such tiles wait for one load
// instead of two.  6144 x 24576 with dense escape bands: 55.3 -> 52.6 us;
// N(0, 0.015): 47.8 -> 47.3.  K15 (more instructions per tile: banded 60.3 ->
// 62.9 us), batch 4 and short waves (14336 x 4096, 4 tiles per wave: 25.2 ->
// 27.7 us) measured slower with them.
#ifndef WC_RING_BIG
#define WC_RING_BIG 1
#endif
constexpr uint32_t kRingBigSlotDwords = 1288;  // 3072 + 2048 + 32 bytes
static bool ring_big_slots(int layout, uint32_t batch, uint64_t waves, uint64_t tiles_per_wave) {
  return WC_RING_BIG && layout == WC_LAYOUT_BYTESPLIT && batch == 1 && tiles_per_wave >= 8 &&
         waves > (uint64_t)cu_count() * 16u;
}

template <int LAYOUT, bool CMP>
static void launch_fused_fast(const GemvArgs& a0, hipStream_t s) {
  GemvArgs a = a0;
  a.rows_per_wave = rows_per_wave(a.rows, a.cols);
  // Batch sizes 1, 2, 3, 4, 8 and 16 have their own kernels; other sizes run
  // as a sum of those over consecutive slices of x and y.
  uint32_t done = 0;
  while (done < a.batch) {
    const uint32_t left = a.batch - done;
    GemvArgs p = a;
    p.x = a.x + (uint64_t)done * a.cols;
    p.y = a.y + (uint64_t)done * a.rows;
    uint32_t b = left >= 16 ? 16 : left >= 8 ? 8 : left >= 4 ? 4 : left;
    p.batch = b;
    const dim3 g = wave_grid(a.rows, a.rows_per_wave), t(kBlockThreads);
    // (batches of 8 and 16 with whole-tile rows take the matrix-core kernel)
    if (kGemvRing && a.cols % kTile == 0 && b <= 4) {
      // Batches 3 and 4 on rows of more than kSplitMinTiles tiles: each row
      // split into 2 parts of whole tiles, one wave each (see the kernel).
      // Two parts measured faster than four (6144 x 24576 banded, batch 4:
      // 85.3 -> 82.7 us byte-split, 86.8 -> 84.9 K15; N(0, 0.015) K15 85.5 ->
      // 81.5) and, at batch 3, than whole rows (banded 76.3 -> 72.0, 79.5 ->
      // 74.3); at batches 1 and 2, in 4-wave blocks, they cost 3-7% on
      // tensors without dense escape rows.
      // K15 at batch 1 splits escape-rich tensors (more than one weight in
      // 32), whose dense rows make long waves: 6144 x 24576 banded 56.7 ->
      // 55.7 us. Byte-split there keeps whole rows in the large ring slots
      // (50.5 us whole, 54.3 split).
      const uint64_t tpr = a.cols / kTile;
      // Byte-split at batch 2 splits too, in 8-wave blocks (6144 x 24576
      // N(0, 0.015) 56.3 -> 54.5 us, banded 1-4% faster in two runs; K15 the
      // same or slower there).
      const bool split_b = b == 4 || b == 3 || (b == 2 && LAYOUT == WC_LAYOUT_BYTESPLIT) ||
                           (LAYOUT == WC_LAYOUT_K15 && b == 1 && 32u * a.n_esc > a.rows * a.cols);
      const uint32_t wpr = split_b && tpr > kSplitMinTiles && tpr % 2 == 0 ? 2u : 1u;
      const uint64_t waves = (a.rows + a.rows_per_wave - 1) / a.rows_per_wave;
      if (wpr > 1) {
        GemvArgs v = p;
        v.wpr = wpr;
        v.x_cols = a.cols;
        v.rows = a.rows * wpr;
        v.cols = a.cols / wpr;
        v.rows_per_wave = 1;
        // Batches 2 to 4 in blocks of 8 waves (4 rows, part-major: the 4
        // waves of a part read the same x columns), except K15 with more
        // than one weight in 32 escaping, whose slow dense rows would hold
        // twice the LDS until their block ends.  6144 x 24576 byte-split:
        // banded batch 4 82.6 -> 81.6 us (batch 3 the same); N(0, 0.015)
        // batch 3 69.2 -> 65.3; K15 N(0, 0.015) batch 4 81.7 -> 79.5, batch 3
        // 70.4 -> 68.5; K15 banded batch 4 85.0 -> 86.6 (kept at 4).
        // (a block must hold whole rows: wpr divides its wave count)
        const bool eight = b >= 2 && 8u % wpr == 0 &&
                           (LAYOUT == WC_LAYOUT_BYTESPLIT || 32u * a.n_esc <= a.rows * a.cols);
        const dim3 g8((unsigned)((v.rows + 7) / 8)), t8(8 * kWave);
        if (b == 4 && eight)
          hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 4, CMP, true, kRingSlotDwords, 8>), g8, t8, 0, s, v);
        else if (b == 3 && eight)
          hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 3, CMP, true, kRingSlotDwords, 8>), g8, t8, 0, s, v);
        else if (b == 2 && eight)
          hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 2, CMP, true, kRingSlotDwords, 8>), g8, t8, 0, s, v);
        else if (b == 4)
          hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 4, CMP, true>), wave_grid(v.rows, 1), t, 0, s, v);
        else if (b == 3)
          hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 3, CMP, true>), wave_grid(v.rows, 1), t, 0, s, v);
        else if (b == 2)
          hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 2, CMP, true>), wave_grid(v.rows, 1), t, 0, s, v);
        else
          hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 1, CMP, true>), wave_grid(v.rows, 1), t, 0, s, v);
      } else if (ring_big_slots(LAYOUT, b, waves, a.rows_per_wave * tpr)) {
        if constexpr (LAYOUT == WC_LAYOUT_BYTESPLIT)
          hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 1, CMP, false, kRingBigSlotDwords>), g, t, 0, s, p);
      } else {
        switch (b) {
          case 4: hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 4, CMP, false>), g, t, 0, s, p); break;
          case 3: hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 3, CMP, false>), g, t, 0, s, p); break;
          case 2: hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 2, CMP, false>), g, t, 0, s, p); break;
          default: hipLaunchKernelGGL((k_decode_gemv_ring<LAYOUT, 1, CMP, false>), g, t, 0, s, p); break;
        }
      }
    } else {
      switch (b) {
        case 16: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 16, CMP>), g, t, 0, s, p); break;
        case 8: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 8, CMP>), g, t, 0, s, p); break;
        case 4: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 4, CMP>), g, t, 0, s, p); break;
        case 3: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 3, CMP>), g, t, 0, s, p); break;
        case 2: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 2, CMP>), g, t, 0, s, p); break;
        default: hipLaunchKernelGGL((k_decode_gemv<LAYOUT, 1, CMP>), g, t, 0, s, p); break;
      }
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
  // raw layout: the stored weights are plain BF16
  if (h.layout == WC_LAYOUT_RAW)
    return launch_gemv_bf16((const uint16_t*)(container + h.off_raw), rows, cols, x, batch, y, s);
  if (batch > 16) {
    if (gemm_wide_fits(rows, cols, batch))
      return launch_decode_gemm_mfma(h, container, rows, cols, x, batch, y, s);
    // other shapes: batches of at most 16 rows in turn
    for (uint32_t done = 0; done < batch; done += 16) {
      const uint32_t b = batch - done < 16 ? batch - done : 16;
      const hipError_t e = launch_decode_gemv(h, container, rows, cols, x + (uint64_t)done * cols,
                                              b, y + (uint64_t)done * rows, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // Batch 4 also takes the matrix cores on grids of 384 row blocks or more
  // when fewer than one weight in 64 escapes (6144 x 24576 N(0, 0.015)
  // byte-split: 82.6 -> 77.8 us; 14336 x 4096 byte-split 34.9 -> 31.7); with
  // denser escapes (the banded tensor, K15 at 2%) or on smaller grids
  // (4096 x 4096: 10.8 against 12.5) the LDS ring is faster.
  const bool mfma4 = batch == 4 && rows >= 384u * 16u && 64u * h.n_esc < h.n;
  if ((batch >= kMfmaMinBatch || mfma4) && gemm_mfma_fits(rows, cols, batch))
    return launch_decode_gemm_mfma(h, container, rows, cols, x, batch, y, s);
  GemvArgs a{};
  a.codes = container + h.off_codes;
  a.raw = container + h.off_raw;
  a.esc_pos = (const uint32_t*)(container + h.off_esc_pos);
  a.esc_sym = container + h.off_esc_sym;
  a.esc_idx = (const uint32_t*)(container + h.off_esc_idx);
  a.w = nullptr;
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.n_esc = h.n_esc;
  // with no escapes, the (never used) escape loads read the container header
  a.esc_last = h.n_esc ? h.n_esc - 1 : 0;
  a.sym_last = h.n_esc ? (h.off_esc_idx - h.off_esc_sym) / 4 - 1 : 0;
  if (h.n_esc == 0) {
    a.esc_pos = (const uint32_t*)container;
    a.esc_sym = container;
    a.esc_idx = (const uint32_t*)container;
  }
  a.raw_last = pad16(raw_bytes(h.layout, h.n)) / 4 - 1;
  if (h.flags & WC_FLAG_COMPACT) {
    // no positions: every tile with escapes places its symbols by rank, and
    // the (never used) position prefetch reads the header
    a.compact = 1;
    a.esc_last = 0;
    a.esc_pos = (const uint32_t*)container;
  }
  a.batch = batch;
  a.dict = dict_of(&h);
  if (cols % kGroup == 0) {
    if (h.layout == WC_LAYOUT_K15)
      a.compact ? launch_fused_fast<WC_LAYOUT_K15, true>(a, s)
                : launch_fused_fast<WC_LAYOUT_K15, false>(a, s);
    else
      a.compact ? launch_fused_fast<WC_LAYOUT_BYTESPLIT, true>(a, s)
                : launch_fused_fast<WC_LAYOUT_BYTESPLIT, false>(a, s);
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
  if (batch > 16) {
    if (gemm_wide_fits(rows, cols, batch)) return launch_gemm_bf16_mfma(w, rows, cols, x, batch, y, s);
    for (uint32_t done = 0; done < batch; done += 16) {
      const uint32_t b = batch - done < 16 ? batch - done : 16;
      const hipError_t e = launch_gemv_bf16(w, rows, cols, x + (uint64_t)done * cols, b,
                                            y + (uint64_t)done * rows, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (batch >= kMfmaMinBatchPlain && gemm_mfma_fits(rows, cols, batch))
    return launch_gemm_bf16_mfma(w, rows, cols, x, batch, y, s);
  GemvArgs a = {};
  a.w = w;
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.batch = batch;
  if (cols % kGroup != 0) {
    hipLaunchKernelGGL(k_gemv_bf16_generic, row_grid(rows), dim3(kBlockThreads), 0, s, a);
    return hipGetLastError();
  }
  a.rows_per_wave = rows_per_wave(rows, cols);
  uint32_t done = 0;
  while (done < batch) {
    const uint32_t left = batch - done;
    GemvArgs p = a;
    p.x = x + (uint64_t)done * cols;
    p.y = y + (uint64_t)done * rows;
    uint32_t b = left >= 16 ? 16 : left >= 8 ? 8 : left >= 4 ? 4 : left;
    p.batch = b;
    const dim3 g = wave_grid(rows, a.rows_per_wave), t(kBlockThreads);
    switch (b) {
      case 16: hipLaunchKernelGGL(k_gemv_bf16<16>, g, t, 0, s, p); break;
      case 8: hipLaunchKernelGGL(k_gemv_bf16<8>, g, t, 0, s, p); break;
      case 4: hipLaunchKernelGGL(k_gemv_bf16<4>, g, t, 0, s, p); break;
      case 3: hipLaunchKernelGGL(k_gemv_bf16<3>, g, t, 0, s, p); break;
      case 2: hipLaunchKernelGGL(k_gemv_bf16<2>, g, t, 0, s, p); break;
      default: hipLaunchKernelGGL(k_gemv_bf16<1>, g, t, 0, s, p); break;
    }
    done += b;
  }
  return hipGetLastError();
}

}  // namespace wc
