// wc_gemm.hip — decode fused into a batched GEMV on the matrix cores, and the
// plain BF16 kernel of the same shape it is measured against.
//
// Page "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está listo
// para producción?", section "¿Qué significa “sin pérdida” para los pesos de
// un LLM?": the coded weights stay on the GPU and the exact BF16 values are
// rebuilt in registers right before the product.  With several input rows
// (batch up to 16) the product is a skinny GEMM, y[b][r] = sum_c W[r][c]
// x[b][c], and v_mfma_f32_16x16x32_bf16 computes it exactly as the scalar
// definition does (exact BF16 products, fp32 sums) while x is reused by 16
// weight rows at once instead of being re-read from L2 for every row.
//
// Block = 16 consecutive rows x all columns, S waves.  The columns are cut
// into 128-wide chunks; at step q wave s takes chunk q*S + s, so the block
// walks the rows left to right in lock step (escape-heavy tensors with rows
// of 12k whole tiles: wave s takes its own contiguous run of chunks
// instead, see CONTIG below).  Lane l = r + 16 h of a wave
// owns 32 consecutive weights of row r (columns 32h .. 32h+31 of the chunk,
// 4 groups of 8): one 16-byte code load, one 32-byte (byte-split) or 28-byte
// (K15) raw load and one 64-byte load of x row r (batch index r) per step,
// all naturally aligned when cols is a multiple of 32.  For MFMA instance m
// (0..3) the lane gives group m of its weights as operand A (row r) and the
// matching 8 x values as operand B (batch column r): both operands put the
// same column at the same (lane / 16, element) slot, so the 32-term dot
// products are exactly the row-times-x sums over those columns.
//
// Escapes (page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%",
// section "Cómo funciona la compresión"): the records are in position order,
// so the records of a lane's weights are one contiguous run of the stream.
// A chunk's codes arrive two steps before it is multiplied: one step ahead
// every wave counts the code-15 marks of the next chunk per row and the
// waves swap these counts through LDS (not needed with contiguous runs);
// every lane then knows the first record of its own weights there (row
// cursor + counts of the chunks and lanes to its left) and issues the load
// of its run as one window, which arrives with the chunk's raw part and x.
// Each group of 8 weights then takes its symbols by rank from its part of
// that window (v_perm selectors, as in the 1D kernels).  Measured at batch
// 16 against the window loaded within the step: 6144 x 24576 N(0, 0.015)
// byte-split 107.7 -> 100.0 us, banded 118.3 -> 114.0; 4096 x 14336 44.9
// -> 40.5.
// The row cursors start from the escape index: one load for a row that
// starts on a 2048-weight boundary, else a search of the records of the row
// start's index tile.
#include "wc_launch.h"
#include "wc_tile.h"

namespace wc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3a4 __attribute__((ext_vector_type(3), aligned(4)));

constexpr int kMRows = 16;       // rows per block: the MFMA's M (and N = batch)
constexpr int kStepCols = 128;   // columns per wave step
constexpr int kLaneCols = 32;    // weights per lane per step

struct GemmArgs {
  const uint8_t* codes;
  const uint8_t* raw;
  const uint32_t* esc_pos;
  const uint8_t* esc_sym;
  const uint32_t* esc_idx;
  const uint16_t* w;  // plain BF16 weights (comparator)
  const uint16_t* x;
  float* y;
  uint64_t rows, cols, n_esc, sym_last;  // sym_last: last dword of the padded symbol stream
  uint32_t batch, chunks;                // chunks: 128-column chunks per row
  uint32_t groups, row_blocks;           // wide batches: batch groups x column splits, row blocks
  uint32_t splits, split_chunks;         // wide batches: column splits, chunks per split
  uint32_t compact;                      // escape symbols only (no position stream)
  Dict dict;
};

__device__ inline f32x4 mfma_bf16(const uint32_t a[4], const uint32_t b[4], f32x4 c) {
  const u32x4 av = {a[0], a[1], a[2], a[3]};
  const u32x4 bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                 __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
}

// Barrier that orders only LDS: global loads in flight stay in flight.
__device__ inline void block_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Bit 8m + e of the result = bit 4e + 3 of esc[m] (weight e of group m escapes).
__device__ inline uint32_t compress_marks(const uint32_t esc[kLaneGroups]) {
  uint32_t M = 0;
#pragma unroll
  for (int m = 0; m < kLaneGroups; ++m) {
    uint32_t t = esc[m] >> 3;  // bit 4e
    t = (t | (t >> 3)) & 0x03030303u;
    t = (t | (t >> 6)) & 0x000F000Fu;
    t = (t | (t >> 12)) & 0xFFu;
    M |= t << (8 * m);
  }
  return M;
}

// A lane's 32 weights as Lane4: its codes (masked) and its raw part as
// loaded, 32 bytes (byte-split, group m = dwords 2m, 2m+1) or 28 bytes (K15,
// group m's 56 bits from byte 7m).
template <int LAYOUT>
__device__ inline void lane_of_chunk(const uint32_t c[kLaneGroups], uint32_t cmask,
                                     const uint32_t* wr, Lane4& l) {
#pragma unroll
  for (int m = 0; m < kLaneGroups; ++m) {
    l.codes[m] = c[m] & cmask;
    if constexpr (LAYOUT == WC_LAYOUT_K15) {
      const int d = (7 * m) >> 2, sh = ((7 * m) & 3) * 8;
      l.raw[m][0] = __builtin_amdgcn_alignbit(wr[d + 1], wr[d], sh);
      l.raw[m][1] = __builtin_amdgcn_alignbit(d + 2 < 7 ? wr[d + 2] : 0u, wr[d + 1], sh);
    } else {
      l.raw[m][0] = wr[2 * m];
      l.raw[m][1] = wr[2 * m + 1];
    }
  }
}

template <int LAYOUT, bool PLAIN>
struct GemmSlot {
  // a lane's symbol window: 32 symbols + alignment
  static constexpr int kWin = PLAIN ? 1 : (LAYOUT == WC_LAYOUT_K15 ? 17 : 9);
  uint32_t wr[PLAIN ? 16 : (LAYOUT == WC_LAYOUT_K15 ? 7 : 8)];  // raw part, or plain BF16
  uint32_t xv[16];                                             // 32 x values of batch row r
  uint32_t wd[kWin];  // the step's symbol window (fused), loaded a step ahead
  uint32_t woff;      // byte of the lane's first record in wd[0]
};

// CONTIG: wave s takes the contiguous chunks [s * n_steps, (s + 1) * n_steps)
// of its rows instead of every S-th chunk.  Used when each wave's first
// column is a multiple of 2048 in the flat index (cols a multiple of
// 2048 S): every row's cursor is then the escape-index entry at that column,
// and the wave advances it by its own counts, with no exchange between waves.
template <int LAYOUT, bool PLAIN, int S, bool CONTIG>
__global__ __launch_bounds__(kWave * S) void k_gemm_mfma(GemmArgs a) {
  constexpr bool kK15 = LAYOUT == WC_LAYOUT_K15;
  constexpr int kWinDwords = kK15 ? 17 : 9;  // a lane's symbol window: 32 symbols + alignment
  constexpr int kSymBytes = kK15 ? 2 : 1;
  constexpr int kGroupWin = WinDwords<LAYOUT>::value;  // dwords read per group (8 symbols + alignment)
  // a lane's window in LDS, with room for a group's read to run past its end
  constexpr int kWinStride = kWinDwords + kGroupWin - 1;
  __shared__ uint32_t T2[PLAIN ? 1 : 256];
  // Symbols go in by rank from each group's window.  (K15 once inserted
  // sparse escapes one record at a time through an LDS stage instead; with
  // the K15 window placement of wc_tile.h the rank path measured faster:
  // 14336 x 4096 at batch 16, 66.5 -> 53.9 us.)  The stage holds the final
  // sums of the S waves.
  __shared__ __attribute__((aligned(16))) uint32_t stage[S][kWave * 4];
  __shared__ uint32_t win[PLAIN ? 1 : S][PLAIN ? 1 : kWave * kWinStride];
  // escapes per row in each wave's chunk
  __shared__ __attribute__((aligned(16))) uint32_t xcnt[2][kMRows][S];
  __shared__ uint64_t erow0[kMRows];
  if constexpr (!PLAIN) build_pair_table<LAYOUT>(T2, a.dict);

  const int lane = lane_id(), r = lane & 15, h = lane >> 4;
  const int s = wave_in_block();
  const uint64_t r0 = (uint64_t)blockIdx.x * kMRows;
  const bool row_ok = r0 + r < a.rows;
  // Lane l feeds x row r (batch column r of the product); lanes past the
  // batch re-read row 0, and their output columns are dropped.
  const bool x_ok = (uint32_t)r < a.batch;
  const uint32_t n_steps = CONTIG ? a.chunks / S : (a.chunks + S - 1) / S;
  // the chunk (128 columns of the block's rows) this wave takes at step q
  auto chunk_of = [&](uint32_t q) -> uint32_t {
    return CONTIG ? (uint32_t)s * n_steps + q : q * S + (uint32_t)s;
  };
  const bool esc = !PLAIN && a.n_esc != 0;


  // Addresses: a wave-uniform base (the block's first row, the step's
  // chunk) plus a per-lane 32-bit offset (row r, columns 32h), so every load
  // is a scalar base + vector offset.  Lanes whose columns lie past the row
  // end (only in a partial last chunk) or whose row lies past the matrix
  // re-read valid data of their own wave and are masked later.
  const uint32_t r_c = row_ok ? (uint32_t)r : (uint32_t)(a.rows - 1 - r0);
  const uint32_t lane_elt = r_c * (uint32_t)a.cols + (uint32_t)(kLaneCols * h);  // element offset
  const uint32_t lane_elt0 = r_c * (uint32_t)a.cols;                            // columns 0..31
  const uint32_t x_elt = (x_ok ? (uint32_t)r : 0u) * (uint32_t)a.cols + (uint32_t)(kLaneCols * h);
  const uint32_t x_elt0 = (x_ok ? (uint32_t)r : 0u) * (uint32_t)a.cols;
  const uint64_t blk_elt = r0 * a.cols;  // first weight of the block

  // Whether the lane's 32 columns at step q are inside the row.
  auto lane_ok = [&](uint32_t q) -> bool {
    const uint32_t j = chunk_of(q);
    return j < a.chunks && (uint64_t)j * kStepCols + (uint64_t)(kLaneCols * h) < a.cols;
  };

  // Whether the 32-column block u of the step-q chunk is inside the rows
  // (wave-uniform).
  auto block_ok = [&](uint32_t q, int u) -> bool {
    const uint32_t j = chunk_of(q);
    return j < a.chunks && (uint64_t)j * kStepCols + (uint64_t)(32 * u) < a.cols;
  };

  using Slot = GemmSlot<LAYOUT, PLAIN>;
  // Raw part (or plain BF16 weights) and x of step q into `sl`.
  auto load = [&](uint32_t q, Slot& sl) {
    const uint32_t j = chunk_of(q);
    const uint32_t jc = j < a.chunks ? j : a.chunks - 1;
    const bool ok = lane_ok(q);
    const uint64_t base = blk_elt + (uint64_t)jc * kStepCols;  // uniform, a multiple of 32
    const uint32_t le = ok ? lane_elt : lane_elt0;               // multiple of 32
    const uint32_t xe = ok ? x_elt : x_elt0;
    if constexpr (PLAIN) {
      // plain BF16, interleaved: group 4u + h of the chunk for instance u, so
      // each load reads 64 contiguous bytes of every row; a 32-column block
      // past the row end re-reads block 0 (its product is skipped)
      const u32x4* wp = (const u32x4*)(a.w + base);
      const u32x4* xq = (const u32x4*)(a.x + (uint64_t)jc * kStepCols);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t g = (block_ok(q, u) ? 4u * u : 0u) + (uint32_t)h;
        const u32x4 v = __builtin_nontemporal_load(wp + (lane_elt0 / 8 + g));
        sl.wr[4 * u] = v[0]; sl.wr[4 * u + 1] = v[1]; sl.wr[4 * u + 2] = v[2]; sl.wr[4 * u + 3] = v[3];
        const u32x4 xv = *(xq + (x_elt0 / 8 + g));
        sl.xv[4 * u] = xv[0]; sl.xv[4 * u + 1] = xv[1]; sl.xv[4 * u + 2] = xv[2]; sl.xv[4 * u + 3] = xv[3];
      }
      return;
    } else {
      if constexpr (kK15) {
        const uint32_t* rp = (const uint32_t*)(a.raw + 7 * (base / 8)) + 7 * (le / 32);  // 28 bytes
        const u32x4 v0 = __builtin_nontemporal_load((const u32x4a4*)rp);
        const u32x3 v1 = __builtin_nontemporal_load((const u32x3a4*)(rp + 4));
        sl.wr[0] = v0[0]; sl.wr[1] = v0[1]; sl.wr[2] = v0[2]; sl.wr[3] = v0[3];
        sl.wr[4] = v1[0]; sl.wr[5] = v1[1]; sl.wr[6] = v1[2];
      } else {
        const u32x4* rp = (const u32x4*)(a.raw + base) + le / 16;
        const u32x4 v0 = __builtin_nontemporal_load(rp), v1 = __builtin_nontemporal_load(rp + 1);
        sl.wr[0] = v0[0]; sl.wr[1] = v0[1]; sl.wr[2] = v0[2]; sl.wr[3] = v0[3];
        sl.wr[4] = v1[0]; sl.wr[5] = v1[1]; sl.wr[6] = v1[2]; sl.wr[7] = v1[3];
      }
    }
    const u32x4* xp = (const u32x4*)(a.x + (uint64_t)jc * kStepCols) + xe / 8;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x4 v = *(xp + u);
      sl.xv[4 * u] = v[0]; sl.xv[4 * u + 1] = v[1]; sl.xv[4 * u + 2] = v[2]; sl.xv[4 * u + 3] = v[3];
    }
  };
  // Codes of step q (fused), loaded two steps ahead of their rebuild.
  auto load_codes = [&](uint32_t q, uint32_t c[kLaneGroups]) {
    const uint32_t j = chunk_of(q);
    const uint32_t jc = j < a.chunks ? j : a.chunks - 1;
    const uint64_t base = blk_elt + (uint64_t)jc * kStepCols;
    // (an offset, not a choice between the two captured values: the
    // optimizer turns that into a pointer select that keeps the closure,
    // and what it refers to, in scratch memory)
    const uint32_t le = lane_elt0 + (lane_ok(q) ? (uint32_t)(kLaneCols * h) : 0u);
    const u32x4 cv = __builtin_nontemporal_load((const u32x4*)(a.codes + base / 2) + le / 32);
    c[0] = cv[0]; c[1] = cv[1]; c[2] = cv[2]; c[3] = cv[3];
  };

  uint64_t e_row = 0;  // escape cursor of row r: the first record of the next chunk counted

  // The first record of the lane's weights in step q's chunk (row cursor +
  // escapes of the chunks and lanes to its left), and the lane's escape
  // count; advances the row cursors past the chunk.  Codes of lanes outside
  // the rows count no escapes.
  auto cursor = [&](uint32_t q, const uint32_t c[kLaneGroups], uint32_t& cnt) -> uint64_t {
    const uint32_t cmask = (lane_ok(q) && row_ok) ? ~0u : 0u;
    Lane4 l;
#pragma unroll
    for (int m = 0; m < kLaneGroups; ++m) l.codes[m] = c[m] & cmask;
    uint32_t marks[kLaneGroups];
    escape_marks(l, marks);
    cnt = count_marks(marks);
    // escapes of this row in the lanes to the left (same wave), and the row's total
    const uint32_t c0 = __shfl(cnt, r, kWave), c1 = __shfl(cnt, r + 16, kWave);
    const uint32_t c2 = __shfl(cnt, r + 32, kWave), c3 = __shfl(cnt, r + 48, kWave);
    const uint32_t ex = (h > 0 ? c0 : 0u) + (h > 1 ? c1 : 0u) + (h > 2 ? c2 : 0u);
    uint32_t pre = 0, tot = c0 + c1 + c2 + c3;
    if constexpr (!CONTIG) {
      // the chunks of other waves lie between this wave's: swap counts
      if (h == 0) xcnt[q & 1][r][s] = tot;
      block_lds_barrier();
      tot = 0;
#pragma unroll
      for (int t = 0; t < S; ++t) {
        const uint32_t v = xcnt[q & 1][r][t];
        pre += t < s ? v : 0u;
        tot += v;
      }
    }
    const uint64_t e_l = e_row + pre + ex;
    e_row += tot;
    return e_l;
  };
  // Symbol window of a lane with escapes: the dwords holding records e_l ..
  // e_l + 31, its end clamped to the stream's padded end (its start may then
  // fall in the preceding streams of the container, which is harmless).
  auto load_window = [&](uint64_t e_l, uint32_t cnt, Slot& sl) {
    if constexpr (!PLAIN) {
      const int64_t byte = (int64_t)(e_l * kSymBytes);
      int64_t b = byte >> 2;
      const int64_t bmax = (int64_t)a.sym_last - (kWinDwords - 1);
      b = b < bmax ? b : bmax;
      sl.woff = (uint32_t)(byte - 4 * b);
      if (cnt != 0) {
        const uint32_t* sp = (const uint32_t*)a.esc_sym + b;
#pragma unroll
        for (int u = 0; u + 4 <= kWinDwords; u += 4) {
          const u32x4 v = *(const u32x4a4*)(sp + u);
          sl.wd[u] = v[0]; sl.wd[u + 1] = v[1]; sl.wd[u + 2] = v[2]; sl.wd[u + 3] = v[3];
        }
        sl.wd[kWinDwords - 1] = sp[kWinDwords - 1];
      }
    }
  };

  // One step (fused): issue step q+1's raw part and x; rebuild the lane's
  // 32 weights of step q; issue step q+2's codes into the registers step q's
  // codes held; count step q+1's escapes and issue its symbol windows; patch
  // step q's escapes from the windows loaded during the previous step;
  // multiply.  Every load is thus issued a step (codes: two) before its use.
  // (Issuing the windows after the patch, so that two steps' windows are not
  // held at once, saves registers but measured slower: 6144 x 24576 at
  // batch 16, 120 against 114 us.)
  // Plain: issue step q+1's loads, multiply.
  // (always inlined: its slots and code arrays must stay in registers)
  auto step = [&](uint32_t q, Slot& cur, Slot& nxt, uint32_t cq[kLaneGroups],
                  const uint32_t cq1[kLaneGroups], f32x4& acc) __attribute__((always_inline)) {
    const bool ok = lane_ok(q);
    // Every lane of the wave is inside its row unless the chunk is the
    // row's partial last one or lies past it (a wave-uniform test); lanes
    // outside contribute zero weights and zero x.
    const bool full = (uint64_t)(chunk_of(q) + 1) * kStepCols <= a.cols;
    const uint32_t cmask = (ok && row_ok) ? ~0u : 0u;  // codes of rows past the end count no escapes
    load(q + 1, nxt);
    uint32_t wv[16];
    if constexpr (!PLAIN) {
      uint32_t M = 0;
      {
        Lane4 lr;
        lane_of_chunk<LAYOUT>(cq, cmask, cur.wr, lr);
        if (esc) {
          uint32_t marks[kLaneGroups];
          escape_marks(lr, marks);
          M = compress_marks(marks);
        }
        rebuild_lane<LAYOUT>(T2, lr, wv);
      }
      load_codes(q + 2, cq);
      if (esc) {
        uint32_t cnt1;
        const uint64_t e_l1 = cursor(q + 1, cq1, cnt1);
        load_window(e_l1, cnt1, nxt);
        if (__ballot(M != 0)) {
          uint32_t* wl = win[s] + lane * kWinStride;
          if (M != 0) {
#pragma unroll
            for (int u = 0; u < kWinDwords; ++u) wl[u] = cur.wd[u];
          }
          wave_lds_sync();
          // Group m's records start fm records into the lane's window (fm =
          // the escapes of groups 0 .. m-1): read the dwords from the one
          // holding its first symbol, and place its symbols by rank into
          // the zero placeholders (as the 1D kernels' dense tiles do).
          uint32_t fm = 0;
#pragma unroll
          for (int m = 0; m < kLaneGroups; ++m) {
            const uint32_t gm = (M >> (8 * m)) & 0xFFu;
            if (__ballot(gm != 0)) {
              const uint32_t o = cur.woff + fm * kSymBytes;  // inside the lane's window
              const uint32_t ad = lds_addr(wl) + (o & ~3u);
              uint32_t w[kGroupWin];
              if constexpr (kGroupWin == 3) {
                asm volatile("ds_read_b32 %0, %3\n\tds_read_b32 %1, %3 offset:4\n\tds_read_b32 %2, %3 offset:8\n\t"
                             "s_waitcnt lgkmcnt(0)"
                             : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]) : "v"(ad) : "memory");
              } else {
                asm volatile("ds_read_b32 %0, %5\n\tds_read_b32 %1, %5 offset:4\n\tds_read_b32 %2, %5 offset:8\n\t"
                             "ds_read_b32 %3, %5 offset:12\n\tds_read_b32 %4, %5 offset:16\n\ts_waitcnt lgkmcnt(0)"
                             : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4])
                             : "v"(ad) : "memory");
              }
              if (gm) expand_window<LAYOUT>(gm, w, o & 3u, wv + 4 * m);
            }
            fm += (uint32_t)__popc(gm);
          }
          wave_lds_sync();  // the window is rewritten at the next step
        }
      }
    }
    // Operands of blocks past the row end are zeroed in place with masks
    // rather than skipped, so the four products are issued on every path (no
    // branch joins between matrix-core results).
    uint32_t* wsrc = PLAIN ? cur.wr : wv;
    if (!full) {
#pragma unroll
      for (int m = 0; m < kLaneGroups; ++m) {
        const uint32_t km = PLAIN ? (block_ok(q, m) ? ~0u : 0u) : (ok ? ~0u : 0u);
#pragma unroll
        for (int k = 4 * m; k < 4 * m + 4; ++k) {
          wsrc[k] &= km;
          cur.xv[k] &= km;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kLaneGroups; ++m) acc = mfma_bf16(wsrc + 4 * m, cur.xv + 4 * m, acc);
  };

  // Two register sets alternate, each with its own accumulator (so no
  // accumulator is copied inside the loop); an odd last step runs after the
  // loop, so no path leaves the loop body half-way (which would make the
  // compiler wait for the prefetch at the loop head).  The codes of steps q
  // and q+1 sit in cA and cB (cA then takes step q+2's).
  f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
  Slot s0, s1;
  uint32_t cA[kLaneGroups], cB[kLaneGroups];
  load(0, s0);  // in flight while the row cursors are read
  if constexpr (!PLAIN) {
    load_codes(0, cA);
    load_codes(1, cB);
  }
  if constexpr (CONTIG) {
    // Row cursors at this wave's first column: lane rr reads row rr's
    // escape-index entry (rows past the matrix read the closing entry).
    uint32_t v = 0;
    if (esc && lane < kMRows) {
      const uint64_t row = r0 + (uint64_t)lane;
      const uint64_t last = a.rows * a.cols / WC_INDEX_TILE;
      const uint64_t t = row < a.rows
                             ? (row * a.cols + (uint64_t)s * n_steps * kStepCols) / WC_INDEX_TILE
                             : last;
      const uint32_t x = a.esc_idx[t < last ? t : last];
      v = x < a.n_esc ? x : (uint32_t)a.n_esc;
    }
    e_row = (uint32_t)__shfl((int)v, r, kWave);
    block_lds_barrier();  // pair table (the first loads stay in flight)
  } else {
    // Row cursors: first record at or after each row's start.
    if (esc) {
      for (int rr = s; rr < kMRows; rr += S) {
        const uint64_t t = r0 + rr < a.rows ? (r0 + rr) * a.cols : a.rows * a.cols;
        const uint64_t e = escape_cursor_at(a.compact, a.esc_idx, a.esc_pos, a.codes, a.n_esc,
                                            a.rows * a.cols, t);
        if (lane == 0) erow0[rr] = e;
      }
    }
    block_lds_barrier();  // pair table and cursors (the first loads stay in flight)
    e_row = esc ? erow0[r] : 0;
  }
  if (esc) {
    // step 0's windows
    uint32_t cnt0;
    const uint64_t e_l0 = cursor(0, cA, cnt0);
    load_window(e_l0, cnt0, s0);
  }
  for (uint32_t q = 0; q + 1 < n_steps; q += 2) {
    step(q, s0, s1, cA, cB, acc0);
    step(q + 1, s1, s0, cB, cA, acc1);
  }
  if (n_steps & 1u) step(n_steps - 1, s0, s1, cA, cB, acc0);
  // Matrix-core results are read by vector instructions only after this
  // many idle cycles (more than the longest product needs to retire).
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc0), "+v"(acc1));
  const f32x4 acc = acc0 + acc1;

  // Sum the S waves' partial tiles.  Lane l holds rows 4h .. 4h+3 of the
  // block for batch column r.
  float* red = (float*)stage[0];
  block_lds_barrier();
  *((f32x4*)(red + 4 * (s * kWave + lane))) = acc;
  block_lds_barrier();
  if (s == 0) {
    f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < S; ++u) t += *((const f32x4*)(red + 4 * (u * kWave + lane)));
    if (x_ok) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint64_t row = r0 + 4 * h + v;
        if (row < a.rows) a.y[(uint64_t)r * a.rows + row] = t[v];
      }
    }
  }
}

// ---- wide batches (17 .. 256) ---------------------------------------------
//
// The prefill-like regime: more input rows than one MFMA's 16 columns.  The
// rebuilt weights are the product's A operand as above, but now every A
// operand is used by NB batch tiles of 16, so a weight is decoded once per
// group of 16 NB batch rows instead of once per 16.
//
// Block = NW waves x 16 rows each, for one group of NB batch tiles.  Each
// wave walks all columns of its own 16 rows, 128 at a time, so its row
// cursors advance by its own escape counts alone.  The block's x chunk (16 NB
// batch rows x 128 columns, 4 KiB per tile) is staged in LDS by global->LDS
// DMA and read by all NW waves: piece p (columns 8p .. 8p+7) of tile row q
// sits at slot p ^ q of that row, so the 16 rows of an operand read fall in
// 16 different bank groups.
//
// Pipeline: at step j the wave has chunk j's raw part, x chunk and symbol
// window and chunk j+1's codes in hand.  It counts chunk j+1's escapes at
// once (so its records' cursors are known a step early), issues chunk j+1's
// window, x, raw loads and chunk j+2's codes, then rebuilds and multiplies
// chunk j.  Every load is thus issued a full step before it is used and the
// step never waits on memory in the middle.
// Operand B of NB batch tiles (16-byte LDS reads 4096 bytes apart from
// addr) behind one wait.  Hand-written: the compiler cannot tell these reads
// from the x chunk that global->LDS loads are still filling for the next
// step, and before a plain read it would wait for all of those loads.
template <int NB>
__device__ inline void lds_read_tiles(uint32_t addr, u32x4 (&v)[NB]) {
  static_assert(NB == 2 || NB == 4 || NB == 8, "batch tiles per block");
  if constexpr (NB == 8) {
    lds_read_tiles<4>(addr, *reinterpret_cast<u32x4(*)[4]>(&v[0]));
    lds_read_tiles<4>(addr + 16384u, *reinterpret_cast<u32x4(*)[4]>(&v[4]));
  } else if constexpr (NB == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:4096\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(addr) : "memory");
  } else {
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:4096\n\t"
                 "ds_read_b128 %2, %4 offset:8192\n\tds_read_b128 %3, %4 offset:12288\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(addr) : "memory");
  }
}

// Weight-stream loads of the wide kernel.  The batch groups of one row
// block read the same weights on one XCD (see the block mapping), so those
// loads keep the default cache policy where the second group then finds the
// lines in L2: byte-split and plain BF16 on the 6144 x 24576 banded tensor
// at batch 256 fetch 30% less from HBM (332 against 338 us byte-split).
// K15, whose symbol windows compete for the same L2, measured slower that
// way (457 against 436 us) and keeps non-temporal loads.
template <bool NT, typename T>
__device__ inline T wide_load(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <int LAYOUT, bool PLAIN, int NW, int NB, int U>
__global__ __launch_bounds__(kWave * NW) void k_gemm_wide(GemmArgs a) {
  constexpr bool kK15 = LAYOUT == WC_LAYOUT_K15;
  constexpr int kRawDw = PLAIN ? 16 : (kK15 ? 7 : 8);  // raw part (or plain weights) per lane
  constexpr int kWinDwords = kK15 ? 17 : 9;
  constexpr int kSymBytes = kK15 ? 2 : 1;
  constexpr int kGroupWin = WinDwords<LAYOUT>::value;
  constexpr int kWinStride = kWinDwords + kGroupWin - 1;
  constexpr int kXTile = kMRows * kStepCols * 2;  // bytes of one batch tile's x chunk
  constexpr int kXChunk = NB * kXTile;            // the block's x for one chunk
  static_assert((4 * NB) % NW == 0, "x DMA split");
  __shared__ uint32_t T2[PLAIN ? 1 : 256];
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][U * kXChunk];
  __shared__ uint32_t win[PLAIN ? 1 : NW][PLAIN ? 1 : kWave * kWinStride];

  // Block -> (row block, batch group).  Workgroups go to the 8 XCDs in turn,
  // so the groups of one row block are given consecutive slots of one XCD:
  // their weight reads then meet in that XCD's L2.
  const uint32_t L = blockIdx.x, xcd = L & 7u, li = L >> 3;
  const uint32_t rb = (li / a.groups) * 8u + xcd, bgs = li % a.groups;
  if (rb >= a.row_blocks) return;  // padding of the grid to whole XCD rounds
  // column split sk takes chunks [c0, c0 + n_chunks) of the block's rows
  const uint32_t sk = bgs % a.splits, bg = bgs / a.splits;
  const uint32_t c0 = sk * a.split_chunks;
  if (c0 >= a.chunks) return;
  const uint32_t n_chunks = a.chunks - c0 < a.split_chunks ? a.chunks - c0 : a.split_chunks;
  const uint64_t col0 = (uint64_t)c0 * kStepCols;
  if constexpr (!PLAIN) build_pair_table<LAYOUT>(T2, a.dict);

  const int lane = lane_id(), r = lane & 15, h = lane >> 4;
  const int s = wave_in_block();
  const uint64_t r0 = ((uint64_t)rb * NW + (uint64_t)s) * kMRows;  // the wave's first row
  const bool row_ok = r0 + r < a.rows;
  // rows past the matrix re-read its last row; their codes count no escapes
  // and their outputs are dropped
  const uint64_t lane_base =
      (row_ok ? r0 + r : a.rows - 1) * a.cols + col0 + (uint64_t)(kLaneCols * h);
  const uint32_t cmask = row_ok ? ~0u : 0u;
  const uint32_t b0 = bg * (uint32_t)(kMRows * NB);
  const uint32_t n_steps = (n_chunks + U - 1) / U;
  const bool esc = !PLAIN && a.n_esc != 0;

  auto load_codes = [&](uint32_t j, uint32_t c[kLaneGroups]) {
    const uint64_t e = lane_base + (uint64_t)j * kStepCols;
    const u32x4 v = wide_load<kK15>((const u32x4*)(a.codes + e / 2));
    c[0] = v[0]; c[1] = v[1]; c[2] = v[2]; c[3] = v[3];
  };
  auto load_raw = [&](uint32_t j, uint32_t w[kRawDw]) {
    const uint64_t e = lane_base + (uint64_t)j * kStepCols;
    if constexpr (PLAIN) {
      const u32x4* wp = (const u32x4*)(a.w + e);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u32x4 v = wide_load<kK15>(wp + u);
        w[4 * u] = v[0]; w[4 * u + 1] = v[1]; w[4 * u + 2] = v[2]; w[4 * u + 3] = v[3];
      }
    } else if constexpr (kK15) {
      const uint32_t* rp = (const uint32_t*)(a.raw + 7 * (e / 8));  // 28 bytes, 4-aligned
      // (non-temporal, as wide_load takes K15 loads; called directly so the
      // pointer types keep their 4-byte alignment)
      const u32x4 v0 = __builtin_nontemporal_load((const u32x4a4*)rp);
      const u32x3 v1 = __builtin_nontemporal_load((const u32x3a4*)(rp + 4));
      w[0] = v0[0]; w[1] = v0[1]; w[2] = v0[2]; w[3] = v0[3];
      w[4] = v1[0]; w[5] = v1[1]; w[6] = v1[2];
    } else {
      const u32x4* rp = (const u32x4*)(a.raw + e);
      const u32x4 v0 = wide_load<kK15>(rp), v1 = wide_load<kK15>(rp + 1);
      w[0] = v0[0]; w[1] = v0[1]; w[2] = v0[2]; w[3] = v0[3];
      w[4] = v1[0]; w[5] = v1[1]; w[6] = v1[2]; w[7] = v1[3];
    }
  };
  // The block's x chunk j into dst: 4 NB DMA loads of 1 KiB, NW-way split.
  // Load i fills tile i / 4, rows 4 (i % 4) .. +3; lane (r, h) writes slot r
  // of row q = 4 (i % 4) + h with piece r ^ q.  Batch rows past the batch
  // re-read its last row (their outputs are dropped).
  auto load_x = [&](uint32_t j, uint8_t* dst) {
#pragma unroll
    for (int k = 0; k < 4 * NB / NW; ++k) {
      const int i = s + k * NW;
      const int q = 4 * (i & 3) + h;
      uint32_t bb = b0 + (uint32_t)(kMRows * (i >> 2) + q);
      bb = bb < a.batch ? bb : a.batch - 1;
      const uint16_t* src =
          a.x + (uint64_t)bb * a.cols + col0 + (uint64_t)j * kStepCols + 8u * (uint32_t)(r ^ q);
      lds_dma16_keep(src, (uint32_t*)(dst + 1024 * i));  // x: read by the other batch groups' blocks too
    }
  };

  // Escape bookkeeping of one chunk, from its codes: the lane's marks
  // (compressed), and its symbol window, loaded into wd when the wave has any
  // escapes (off = byte of the lane's first symbol in wd).  e_next is row
  // r's cursor at the chunk's first column and moves past the chunk.
  uint64_t e_next = 0;
  auto count_chunk = [&](const uint32_t c[kLaneGroups], uint32_t& M, uint32_t& off, bool& any,
                         uint32_t wd[kWinDwords]) {
    Lane4 l;
#pragma unroll
    for (int m = 0; m < kLaneGroups; ++m) l.codes[m] = c[m] & cmask;
    uint32_t marks[kLaneGroups];
    escape_marks(l, marks);
    const uint32_t cnt = count_marks(marks);
    M = compress_marks(marks);
    const uint32_t c0 = __shfl(cnt, r, kWave), c1 = __shfl(cnt, r + 16, kWave);
    const uint32_t c2 = __shfl(cnt, r + 32, kWave), c3 = __shfl(cnt, r + 48, kWave);
    const uint32_t ex = (h > 0 ? c0 : 0u) + (h > 1 ? c1 : 0u) + (h > 2 ? c2 : 0u);
    const uint64_t e_l = e_next + ex;
    e_next += c0 + c1 + c2 + c3;
    any = __ballot(cnt != 0) != 0;
    off = 0;
    if (any) {
      // the dwords holding records e_l .. e_l+31, the window's end clamped to
      // the stream's padded end (its start may then fall in the container's
      // earlier streams, which is harmless)
      const int64_t byte = (int64_t)(e_l * kSymBytes);
      int64_t b = byte >> 2;
      const int64_t bmax = (int64_t)a.sym_last - (kWinDwords - 1);
      b = b < bmax ? b : bmax;
      off = (uint32_t)(byte - 4 * b);
      if (cnt != 0) {
        const uint32_t* sp = (const uint32_t*)a.esc_sym + b;
#pragma unroll
        for (int u = 0; u + 4 <= kWinDwords; u += 4) {
          const u32x4 v = *(const u32x4a4*)(sp + u);
          wd[u] = v[0]; wd[u + 1] = v[1]; wd[u + 2] = v[2]; wd[u + 3] = v[3];
        }
        wd[kWinDwords - 1] = sp[kWinDwords - 1];
      }
    }
  };

  // Row cursors at column col0: lane rr of the first 16 reads row rr's index
  // entry when those columns start index tiles, else each row is searched
  // for.
  if (esc) {
    if (a.cols % WC_INDEX_TILE == 0 && col0 % WC_INDEX_TILE == 0) {
      uint32_t v = 0;
      if (lane < kMRows) {
        const uint64_t row = r0 + (uint64_t)lane;
        const uint64_t t = row < a.rows ? (row * a.cols + col0) / WC_INDEX_TILE
                                        : a.rows * (a.cols / WC_INDEX_TILE);
        const uint32_t x = a.esc_idx[t];
        v = x < a.n_esc ? x : (uint32_t)a.n_esc;
      }
      e_next = (uint32_t)__shfl((int)v, r, kWave);
    } else {
      for (int rr = 0; rr < kMRows; ++rr) {
        const uint64_t t = r0 + rr < a.rows ? (r0 + rr) * a.cols + col0 : a.rows * a.cols;
        const uint64_t e = escape_cursor_at(a.compact, a.esc_idx, a.esc_pos, a.codes, a.n_esc,
                                            a.rows * a.cols, t);
        if (r == rr) e_next = e;
      }
    }
  }

  // A step takes U consecutive chunks (the last step may hold fewer): their
  // loads go out together, so a block's chain of memory round trips is one
  // per U chunks.
  uint32_t c_cur[U][kLaneGroups] = {}, c_nxt[U][kLaneGroups] = {}, c_new[U][kLaneGroups] = {};
  uint32_t w_cur[U][kRawDw] = {}, w_nxt[U][kRawDw] = {};
  uint32_t wd_cur[U][kWinDwords] = {}, wd_nxt[U][kWinDwords] = {};
  uint32_t M_cur[U] = {}, off_cur[U] = {}, M_nxt[U] = {}, off_nxt[U] = {};
  bool win_cur[U] = {}, win_nxt[U] = {};
  f32x4 acc[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int u = 0; u < U; ++u) {
    if ((uint32_t)u < n_chunks) {
      load_x(u, xs[0] + u * kXChunk);
      load_raw(u, w_cur[u]);
      if constexpr (!PLAIN) load_codes(u, c_cur[u]);
    }
  }
  if constexpr (!PLAIN) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if ((uint32_t)(U + u) < n_chunks) load_codes(U + u, c_nxt[u]);
    if (esc) {
      wait_vm<0>();
#pragma unroll
      for (int u = 0; u < U; ++u)
        if ((uint32_t)u < n_chunks) count_chunk(c_cur[u], M_cur[u], off_cur[u], win_cur[u], wd_cur[u]);
    }
  }

  for (uint32_t j = 0; j < n_steps; ++j) {
    wait_vm<0>();
    if (j > 0) {
      // everything issued last step has arrived: move the ring along (a
      // copy made after the wait, so it never stalls on a load)
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int m = 0; m < kLaneGroups; ++m) { c_cur[u][m] = c_nxt[u][m]; c_nxt[u][m] = c_new[u][m]; }
#pragma unroll
        for (int k = 0; k < kRawDw; ++k) w_cur[u][k] = w_nxt[u][k];
#pragma unroll
        for (int k = 0; k < kWinDwords; ++k) wd_cur[u][k] = wd_nxt[u][k];
        M_cur[u] = M_nxt[u]; off_cur[u] = off_nxt[u]; win_cur[u] = win_nxt[u];
      }
    }
    block_lds_barrier();  // step j's x in LDS for every wave; step j-1's reads done
    const uint32_t q1 = (j + 1) * U, q2 = (j + 2) * U;  // first chunks of the next two steps
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q1 + u < n_chunks) {
        if (esc) count_chunk(c_nxt[u], M_nxt[u], off_nxt[u], win_nxt[u], wd_nxt[u]);
        load_x(q1 + u, xs[(j + 1) & 1] + u * kXChunk);
        load_raw(q1 + u, w_nxt[u]);
        if (!PLAIN && q2 + u < n_chunks) load_codes(q2 + u, c_new[u]);
      }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j * U + u >= n_chunks) continue;  // the last step's missing chunks (uniform)
      uint32_t wv[16];
      if constexpr (PLAIN) {
#pragma unroll
        for (int k = 0; k < 16; ++k) wv[k] = w_cur[u][k];
      } else {
        Lane4 lr;
        lane_of_chunk<LAYOUT>(c_cur[u], cmask, w_cur[u], lr);
        rebuild_lane<LAYOUT>(T2, lr, wv);
        if (win_cur[u]) {
          // each group takes its symbols by rank from its part of the lane's
          // window (written to LDS, where a group's dwords can be addressed)
          uint32_t* wl = win[s] + lane * kWinStride;
          if (M_cur[u] != 0) {
#pragma unroll
            for (int k = 0; k < kWinDwords; ++k) wl[k] = wd_cur[u][k];
          }
          wave_lds_sync();
          uint32_t fm = 0;
#pragma unroll
          for (int m = 0; m < kLaneGroups; ++m) {
            const uint32_t gm = (M_cur[u] >> (8 * m)) & 0xFFu;
            if (__ballot(gm != 0)) {
              const uint32_t o = off_cur[u] + fm * kSymBytes;
              const uint32_t* gp = wl + (o >> 2);
              uint32_t w[kGroupWin];
#pragma unroll
              for (int k = 0; k < kGroupWin; ++k) w[k] = gp[k];
              if (gm) expand_window<LAYOUT>(gm, w, o & 3u, wv + 4 * m);
            }
            fm += (uint32_t)__popc(gm);
          }
          wave_lds_sync();  // the window area is rewritten by the next chunk
        }
      }

      // NB products per group of 8 weights: operand B of tile t is x rows
      // 16 t + r, columns 32 h + 8 m .. +7 of the chunk (piece 4 h + m).
      static_assert(kXTile == 4096, "tile stride of lds_read_tiles");
      const uint32_t xb = lds_addr(xs[j & 1] + u * kXChunk) + 256u * (uint32_t)r;
#pragma unroll
      for (int m = 0; m < kLaneGroups; ++m) {
        u32x4 v[NB];
        lds_read_tiles<NB>(xb + 16u * (uint32_t)((4 * h + m) ^ r), v);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const uint32_t bx[4] = {v[t][0], v[t][1], v[t][2], v[t][3]};
          acc[t] = mfma_bf16(wv + 4 * m, bx, acc[t]);
        }
      }
    }
  }
  // matrix-core results are read by vector instructions only after this
  // many idle cycles
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[0]));
#pragma unroll
  for (int t = 1; t < NB; ++t) asm volatile("" : "+v"(acc[t]));
  // lane (r, h) holds rows 4h .. 4h+3 of the wave's 16 for batch row 16 t + r.
  // With two column splits each output is the sum of two partial sums added
  // into a zeroed y: 0 + p + q and 0 + q + p round to the same value, so the
  // result does not depend on which split finishes first.
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const uint32_t bb = b0 + (uint32_t)(kMRows * t + r);
    if (bb < a.batch) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint64_t row = r0 + 4 * h + v;
        if (row < a.rows) {
          float* yp = a.y + (uint64_t)bb * a.rows + row;
          if (a.splits > 1)
            atomicAdd(yp, acc[t][v]);
          else
            *yp = acc[t][v];
        }
      }
    }
  }
}

// ---- launchers -----------------------------------------------------------

#ifndef WC_GEMM_SLICES
#define WC_GEMM_SLICES 0  // waves per block of the fused kernel: 0 = chosen by grid size
#endif

#ifndef WC_GEMM_PLAIN_SLICES
#define WC_GEMM_PLAIN_SLICES 0  // waves per block of the plain kernel: 0 = chosen by shape
#endif

#ifndef WC_GEMM_CONTIG_SLICES
#define WC_GEMM_CONTIG_SLICES 4
#endif

// Waves per 16-row block.  The fused kernel holds three waves per SIMD (its
// registers), so blocks of 12, 6 or 4 waves pack a compute unit whole.
// Measured at batches 8 and 16 (us at batch 16, 12 / 6 / 4 waves):
// byte-split 4096 x 4096 14.6 / 14.0 / 14.0, 4096 x 14336 40.6 / 40.5 /
// 45.1, 6144 x 24576 banded 116.8 / 114.0 / 116.1, 14336 x 4096 54.7 /
// 54.0 / 40.9; K15 4096 x 4096 18.2 / 18.2 / 19.3, 4096 x 14336 49.6 / 48.7 /
// 53.5, 6144 x 24576 N(0, 0.015) 140.5 / 151.5 / 138.5, 14336 x 4096 67.3 /
// 66.7 / 53.0.  Grids of more than 768 blocks take 2 (14336 x 4096 at
// batch 16: 41.1 -> 38.1 us byte-split, 53.7 -> 51.3 K15; 24576 x 6144:
// 84.7 -> 82.9, 106.6 -> 105.4).  The plain kernel takes 2 waves on grids of
// up to 1024 blocks with rows of up to 16384 columns, else 4 (batch 16:
// 4096 x 4096 11.8 -> 11.2 us, 14336 x 4096 40.4 -> 38.5, 4096 x 14336
// 36.9 -> 34.1; 6144 x 24576 117 against 123 with 2; 8 or 12 waves were
// slower everywhere).
static int mfma_slices(int layout, uint64_t rows) {
  if (WC_GEMM_SLICES) return WC_GEMM_SLICES;
  const uint64_t blocks = (rows + kMRows - 1) / kMRows;
  if (blocks > 768) return 2;
  if (layout == WC_LAYOUT_K15) return blocks <= 256 ? 12 : 4;
  return blocks <= 512 ? 6 : 4;
}

static int mfma_plain_slices(uint64_t rows, uint64_t cols) {
  if (WC_GEMM_PLAIN_SLICES) return WC_GEMM_PLAIN_SLICES;
  const uint64_t blocks = (rows + kMRows - 1) / kMRows;
  return blocks <= 1024 && cols <= 16384 ? 2 : 4;
}

template <int LAYOUT, bool PLAIN>
static void launch_mfma(const GemmArgs& a, hipStream_t s) {
  const dim3 g((unsigned)((a.rows + kMRows - 1) / kMRows));
  constexpr int SC = WC_GEMM_CONTIG_SLICES;
  if constexpr (PLAIN) {
    if (mfma_plain_slices(a.rows, a.cols) == 2)
      hipLaunchKernelGGL((k_gemm_mfma<LAYOUT, true, 2, false>), g, dim3(kWave * 2), 0, s, a);
    else
      hipLaunchKernelGGL((k_gemm_mfma<LAYOUT, true, 4, false>), g, dim3(kWave * 4), 0, s, a);
  } else {
    // K15 whose rows of whole tiles split evenly over SC waves: contiguous
    // per-wave ranges with cursors from the escape index, no count exchange.
    // Measured on the 6144 x 24576 banded tensor (5% escapes) at batch 16:
    // 150 us with 4 waves, 158 with 6 or 12, 158 interleaved; on 6144 x 24576
    // N(0, 0.02) (1.6% escapes) at batch 8: 121 against 128 interleaved
    // (batch 16: 138 either way).  Byte-split is faster interleaved (banded,
    // batch 16: 114 against 126 us with 6 contiguous waves), so it always
    // takes the interleaved ranges.
    if (LAYOUT == WC_LAYOUT_K15 && a.cols % ((uint64_t)WC_INDEX_TILE * SC) == 0) {
      hipLaunchKernelGGL((k_gemm_mfma<LAYOUT, false, SC, true>), g, dim3(kWave * SC), 0, s, a);
      return;
    }
    switch (mfma_slices(LAYOUT, a.rows)) {
      case 12: hipLaunchKernelGGL((k_gemm_mfma<LAYOUT, false, 12, false>), g, dim3(kWave * 12), 0, s, a); break;
      case 6: hipLaunchKernelGGL((k_gemm_mfma<LAYOUT, false, 6, false>), g, dim3(kWave * 6), 0, s, a); break;
      case 2: hipLaunchKernelGGL((k_gemm_mfma<LAYOUT, false, 2, false>), g, dim3(kWave * 2), 0, s, a); break;
      default: hipLaunchKernelGGL((k_gemm_mfma<LAYOUT, false, 4, false>), g, dim3(kWave * 4), 0, s, a); break;
    }
  }
}

static GemmArgs gemm_args(uint64_t rows, uint64_t cols, const uint16_t* x, uint32_t batch,
                          float* y) {
  GemmArgs a = {};
  a.x = x;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.batch = batch;
  a.chunks = (uint32_t)((cols + kStepCols - 1) / kStepCols);
  return a;
}

#ifndef WC_WIDE_NB
#define WC_WIDE_NB 0  // batch tiles per block: 0 = chosen per layout and size
#endif

#ifndef WC_WIDE_U
#define WC_WIDE_U 1
#endif

#ifndef WC_WIDE_NW
#define WC_WIDE_NW 0  // waves per block: 0 = chosen by grid size
#endif

#ifndef WC_WIDE_SPLITS
#define WC_WIDE_SPLITS 2
#endif

// Wide batches: 2, 4 or 8 batch tiles per block, 4 waves (64 rows) per block,
// or 2 when that leaves fewer than two blocks per compute unit.  Eight tiles
// halve the decode work per product and the weight re-reads, at the cost of
// LDS (fewer blocks per compute unit).  Measured (us, 4 vs 8 tiles): K15
// fused on 6144 x 24576 265 -> 225 at batch 64 and 522 -> 462 at 256, but
// 42 -> 49 on 4096 x 4096 at batch 64; byte-split fused 132 -> 155 and
// 288 -> 326 on 6144 x 24576.  The plain kernel, whose batch groups share
// their weight lines in L2, takes 4 (batch 256: 6144 x 24576 banded 302 ->
// 288 us, 4096 x 4096 50 -> 36; 14336 x 4096 103 either way).
static_assert(WC_WIDE_NB == 0 || WC_WIDE_NB == 2 || WC_WIDE_NB == 4 || WC_WIDE_NB == 8,
              "instantiated tile counts");
static_assert(WC_WIDE_NW == 0 || WC_WIDE_NW == 2 || WC_WIDE_NW == 4, "instantiated wave counts");

template <int LAYOUT, bool PLAIN>
static int wide_tiles(const GemmArgs& a) {
  if (WC_WIDE_NB) return WC_WIDE_NB;
  if (PLAIN) return 4;
  // tensors of 2^26 weights or more at batches up to 64: two tiles, so that
  // twice the waves share the decode (6144 x 24576 banded, batch 32: 154 ->
  // 142 us byte-split, 221 -> 204 K15; batch 64: 160 -> 156, 221 -> 211);
  // on 4096 x 4096 two tiles measured slower (batch 64: 31 -> 35 us)
  if (a.batch <= 64 && a.rows * a.cols >= (1ull << 26)) return 2;
  if (LAYOUT == WC_LAYOUT_K15) return a.batch > 64 || a.rows * a.cols >= (1ull << 26) ? 8 : 4;
  return 4;
}

template <int LAYOUT, bool PLAIN>
static void launch_wide(GemmArgs a, hipStream_t s) {
  constexpr int kCUs = 256;
  const int nb = wide_tiles<LAYOUT, PLAIN>(a);
  const uint32_t bgroups = (a.batch + kMRows * nb - 1) / (kMRows * nb);
  const uint64_t rb4 = (a.rows + 4 * kMRows - 1) / (4 * kMRows);
  const int nw = WC_WIDE_NW ? WC_WIDE_NW : (rb4 * bgroups >= 2 * kCUs ? 4 : 2);
  const uint64_t rbs = (a.rows + (uint64_t)nw * kMRows - 1) / ((uint64_t)nw * kMRows);
  // Column splits: each block walks its rows' chunks one after another, so
  // when the grid holds fewer than two blocks per compute unit, two blocks on
  // the two halves of the columns halve that chain (6144 x 24576 at batch
  // 64: 223 -> 134 us byte-split); on a fuller grid the split measured up to
  // 25% slower.  The split point is a whole number of 2048-weight index tiles
  // when the rows are.
  a.splits = WC_WIDE_SPLITS < 2 || a.chunks < 2 || rbs * bgroups >= 2 * kCUs ? 1u : 2u;
  a.split_chunks = a.chunks;
  if (a.splits == 2) {
    uint32_t half = (a.chunks + 1) / 2;
    constexpr uint32_t kTileChunks = WC_INDEX_TILE / kStepCols;
    if (a.cols % WC_INDEX_TILE == 0) half = (half + kTileChunks - 1) / kTileChunks * kTileChunks;
    a.split_chunks = half;
    if (half >= a.chunks) a.splits = 1;
  }
  if (a.splits == 2) {
    const uint64_t count = a.rows * a.batch;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, a.y,
                       count);
  }
  a.groups = bgroups * a.splits;
  a.row_blocks = (uint32_t)rbs;
  const dim3 g((unsigned)(((rbs + 7) / 8) * 8 * a.groups));
  const dim3 t(kWave * nw);
#define WC_WIDE_LAUNCH(NW, NB) \
  hipLaunchKernelGGL((k_gemm_wide<LAYOUT, PLAIN, NW, NB, WC_WIDE_U>), g, t, 0, s, a)
  if (nw == 4 && nb == 2)
    WC_WIDE_LAUNCH(4, 2);
  else if (nb == 2)
    WC_WIDE_LAUNCH(2, 2);
  else if (nw == 4 && nb == 8)
    WC_WIDE_LAUNCH(4, 8);
  else if (nw == 4)
    WC_WIDE_LAUNCH(4, 4);
  else if (nb == 8)
    WC_WIDE_LAUNCH(2, 8);
  else
    WC_WIDE_LAUNCH(2, 4);
#undef WC_WIDE_LAUNCH
}

// The wide kernel's time is set by one memory round trip per 128-column
// step of a block, whatever its batch.  On tensors of 2^26 weights or more it
// beats launches of the 16-row kernel from batch 17 (6144 x 24576 at batch
// 32, byte-split: 129 against 217 us); on 4096 x 4096 only from about batch
// 32, so smaller tensors take it above 32.
#ifndef WC_WIDE_MIN_BATCH
#define WC_WIDE_MIN_BATCH 0  // 0 = by tensor size, as above
#endif

bool gemm_wide_fits(uint64_t rows, uint64_t cols, uint32_t batch) {
  static_assert(WC_WIDE_MIN_BATCH == 0 || WC_WIDE_MIN_BATCH > kMRows,
                "the wide kernel is for batches above 16");
  const uint32_t min_batch = WC_WIDE_MIN_BATCH ? WC_WIDE_MIN_BATCH
                             : rows * cols >= (1ull << 26) ? kMRows + 1 : 2 * kMRows + 1;
  return rows > 0 && cols > 0 && cols % kStepCols == 0 && batch >= min_batch &&
         batch <= WC_MAX_BATCH && cols / kStepCols < (1ull << 31) &&
         rows / (2 * kMRows) < (1ull << 31) / 8;
}

bool gemm_mfma_fits(uint64_t rows, uint64_t cols, uint32_t batch) {
  return rows > 0 && cols > 0 && cols % kLaneCols == 0 && batch >= 1 && batch <= kMRows &&
         cols / kStepCols < (1ull << 31);
}

hipError_t launch_decode_gemm_mfma(const wc_header& h, const uint8_t* container, uint64_t rows,
                                   uint64_t cols, const uint16_t* x, uint32_t batch, float* y,
                                   hipStream_t s) {
  GemmArgs a = gemm_args(rows, cols, x, batch, y);
  a.codes = container + h.off_codes;
  a.raw = container + h.off_raw;
  a.esc_pos = (const uint32_t*)(container + h.off_esc_pos);
  a.esc_sym = container + h.off_esc_sym;
  a.esc_idx = (const uint32_t*)(container + h.off_esc_idx);
  a.n_esc = h.n_esc;
  // last dword of the symbol stream's 16-byte padded extent (unused without escapes)
  a.sym_last = h.n_esc ? (h.off_esc_idx - h.off_esc_sym) / 4 - 1 : 0;
  a.dict = dict_of(&h);
  a.compact = (h.flags & WC_FLAG_COMPACT) ? 1u : 0u;
  if (batch > kMRows) {
    if (h.layout == WC_LAYOUT_K15)
      launch_wide<WC_LAYOUT_K15, false>(a, s);
    else
      launch_wide<WC_LAYOUT_BYTESPLIT, false>(a, s);
  } else if (h.layout == WC_LAYOUT_K15) {
    launch_mfma<WC_LAYOUT_K15, false>(a, s);
  } else {
    launch_mfma<WC_LAYOUT_BYTESPLIT, false>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_mfma(const uint16_t* w, uint64_t rows, uint64_t cols,
                                 const uint16_t* x, uint32_t batch, float* y, hipStream_t s) {
  GemmArgs a = gemm_args(rows, cols, x, batch, y);
  a.w = w;
  if (batch > kMRows)
    launch_wide<WC_LAYOUT_BYTESPLIT, true>(a, s);
  else
    launch_mfma<WC_LAYOUT_BYTESPLIT, true>(a, s);
  return hipGetLastError();
}

}  // namespace wc
