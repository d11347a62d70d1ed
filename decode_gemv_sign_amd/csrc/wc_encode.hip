// wc_encode.hip — per-tensor dictionary and container encode.
//
// Page "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está listo
// para producción?", section "¿Qué demostró realmente el experimento con
// GLM-5.2?": trained weights reuse few sign+exponent combinations, so the
// frequent symbols get short codes and the rare ones an exact escape stream.
// Page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%", section
// "Cómo funciona la compresión": a 4-bit code into a 15-entry table per
// weight; byte-split keeps the low byte, K15 the 7-bit mantissa.
//
// Kernels, in stream order:
//   build_dict: k_zero_hist -> k_hist (512 bins of b >> 7, merged into 8
//               global copies; the byte-split histogram is the pair sum) ->
//               k_top15 (sums the copies; rank by count desc, symbol asc) ->
//               48-byte result copied to the host.
//   encode:     k_pack (codes, raw stream, header and zero gaps, each block's
//               escape count, and the escape symbols of blocks with few
//               escapes staged in the workspace) -> k_scan (exclusive scan of
//               the block counts, one workgroup) -> k_emit (escape positions
//               from the codes and symbols from the stage, in weight order,
//               and the escape index).
// Every output byte is a pure function of the input, so the container is
// byte-identical from run to run.
#include <mutex>

#include "wc_launch.h"
#include "wc_tile.h"

namespace wc {

// ---- histogram -----------------------------------------------------------

// 1024 threads and 32 copies (66 KB of LDS: two workgroups, 32 waves per
// compute unit) on 512 workgroups, one round: 6144 x 24576 in 48.8 us,
// against 55.9 with 256 threads, 16 copies and 1024 workgroups (more waves
// keep more loads in flight; the LDS adds are not what limits it: without
// them the kernel took 52.7 us)
constexpr int kHistThreads = 1024;
constexpr int kHistBlocks = 512;
constexpr int kHistCopies = 32;   // replicated sub-histograms per workgroup
constexpr int kHistStride = 513;  // odd stride: copies of a bin sit in different LDS banks

__global__ void k_zero_hist(uint32_t* hist) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < 512 * kHistGlobal) hist[i] = 0;
}

__global__ __launch_bounds__(kHistThreads) void k_hist(const uint16_t* __restrict__ w, uint64_t n,
                                                        uint32_t* __restrict__ hist) {
  __shared__ uint32_t sub[kHistCopies * kHistStride];
  for (int i = threadIdx.x; i < kHistCopies * kHistStride; i += kHistThreads) sub[i] = 0;
  __syncthreads();
  // lanes spread over the copies, so the few very frequent symbols of a
  // skewed tensor do not serialise on one LDS address
  uint32_t* mine = sub + (lane_id() & (kHistCopies - 1)) * kHistStride;
  const uint64_t stride = (uint64_t)gridDim.x * kHistThreads;
  const uint64_t gid = (uint64_t)blockIdx.x * kHistThreads + threadIdx.x;
  const uint64_t nvec = n / 8;
  const u32x4* wv = (const u32x4*)w;
  // four 16-byte loads in flight per thread, then their 32 symbol counts
  uint64_t v = gid;
  for (; v + 3 * stride < nvec; v += 4 * stride) {
    u32x4 d[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) d[u] = __builtin_nontemporal_load(wv + v + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        atomicAdd(mine + ((d[u][k] >> 7) & 0x1FFu), 1u);
        atomicAdd(mine + (d[u][k] >> 23), 1u);
      }
    }
  }
  for (; v < nvec; v += stride) {
    const u32x4 d = __builtin_nontemporal_load(wv + v);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      atomicAdd(mine + ((d[k] >> 7) & 0x1FFu), 1u);
      atomicAdd(mine + (d[k] >> 23), 1u);
    }
  }
  for (uint64_t i = nvec * 8 + gid; i < n; i += stride) atomicAdd(mine + (w[i] >> 7), 1u);
  __syncthreads();
  // blocks spread their merges over the global copies, so a frequent
  // symbol's bin takes 1/kHistGlobal of the blocks' atomic adds
  uint32_t* const g = hist + 512 * (blockIdx.x % kHistGlobal);
  for (int b = threadIdx.x; b < 512; b += kHistThreads) {
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) s += sub[c * kHistStride + b];
    if (s) atomicAdd(g + b, s);
  }
}

// ---- top-15 --------------------------------------------------------------
// One workgroup of 512 threads, one symbol each.  The symbols that occur are
// first compacted (in symbol order) into a candidate list of m entries; each
// then counts the candidates with a larger count, or an equal count and a
// smaller value: that count is its rank.  Symbols of rank < 15 form the
// dictionary in rank order.  Work is m^2 compares (m is the number of
// distinct symbols, at most 512).

__global__ __launch_bounds__(512) void k_top15(const uint32_t* __restrict__ hist, int layout,
                                               uint64_t n, DictResult* __restrict__ res) {
  __shared__ __attribute__((aligned(16))) uint32_t cand_cnt[512];
  __shared__ uint16_t cand_sym[512];
  __shared__ uint16_t dict[16];
  __shared__ uint32_t wsum[8];
  __shared__ uint32_t wnum[8];
  const int i = threadIdx.x;
  const int wv = i / kWave;
  const int nsym = layout == WC_LAYOUT_K15 ? 512 : 256;
  uint32_t c = 0;
  if (i < nsym) {
#pragma unroll
    for (int k = 0; k < kHistGlobal; ++k) {
      const uint32_t* hk = hist + 512 * k;
      c += layout == WC_LAYOUT_K15 ? hk[i] : hk[2 * i] + hk[2 * i + 1];
    }
  }
  if (i < 16) dict[i] = 0;
  // compact the occurring symbols, keeping symbol order
  const uint32_t occ = c > 0 ? 1u : 0u;
  const uint32_t ex = wave_excl_scan_u32(occ);
  if (lane_id() == kWave - 1) wnum[wv] = ex + occ;
  __syncthreads();
  uint32_t before = 0, m = 0;
  for (int q = 0; q < 8; ++q) {
    before += q < wv ? wnum[q] : 0u;
    m += wnum[q];
  }
  const uint32_t slot = before + ex;
  if (occ) {
    cand_cnt[slot] = c;
    cand_sym[slot] = (uint16_t)i;
  }
  for (uint32_t q = m + (uint32_t)i; q < ((m + 3u) & ~3u); q += 512) cand_cnt[q] = 0;  // pad to 4
  __syncthreads();
  uint32_t rank = 0;
  if (occ) {
    const u32x4* cc4 = (const u32x4*)cand_cnt;
    for (uint32_t j4 = 0; 4 * j4 < m; ++j4) {
      const u32x4 q = cc4[j4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t j = 4 * j4 + (uint32_t)k;
        // candidates before this one in the list have smaller symbols
        rank += (j < m && (q[k] > c || (q[k] == c && j < slot))) ? 1u : 0u;
      }
    }
  }
  const bool in = occ && rank < 15;
  if (in) dict[rank] = (uint16_t)i;
  const uint32_t s = wave_sum_u32(in ? c : 0u);
  const uint32_t k = wave_sum_u32(in ? 1u : 0u);
  __syncthreads();  // wnum is reused below
  if (lane_id() == 0) {
    wsum[wv] = s;
    wnum[wv] = k;
  }
  __syncthreads();
  if (i == 0) {
    uint64_t covered = 0;
    uint32_t nd = 0;
    for (int q = 0; q < 8; ++q) {
      covered += wsum[q];
      nd += wnum[q];
    }
    res->n_dict = nd;
    res->reserved = 0;
    res->n_esc = n - covered;
    for (int q = 0; q < 16; ++q) res->dict[q] = dict[q];
  }
}

hipError_t launch_build_dict(int layout, const uint16_t* w, uint64_t n, uint8_t* work,
                             hipStream_t s) {
  uint32_t* hist = (uint32_t*)(work + kWorkHist);
  hipLaunchKernelGGL(k_zero_hist, dim3(2 * kHistGlobal), dim3(256), 0, s, hist);
  const uint64_t nvec = n / 8;
  uint64_t blocks = (nvec + kHistThreads - 1) / kHistThreads;
  if (blocks > kHistBlocks) blocks = kHistBlocks;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_hist, dim3((unsigned)blocks), dim3(kHistThreads), 0, s, w, n, hist);
  if (layout == WC_LAYOUT_AUTO) {
    hipLaunchKernelGGL(k_top15, dim3(1), dim3(512), 0, s, hist, (int)WC_LAYOUT_BYTESPLIT, n,
                       (DictResult*)(work + kWorkResult));
    hipLaunchKernelGGL(k_top15, dim3(1), dim3(512), 0, s, hist, (int)WC_LAYOUT_K15, n,
                       (DictResult*)(work + kWorkResult2));
  } else {
    hipLaunchKernelGGL(k_top15, dim3(1), dim3(512), 0, s, hist, layout, n,
                       (DictResult*)(work + kWorkResult));
  }
  return hipGetLastError();
}

// ---- pack, scan, escape records ---------------------------------------------
//
// Block b of k_pack and of k_emit covers weights [8192 b, 8192 b + 8192):
// 1024 groups of 8, thread t taking groups t, t+256, t+512, t+768, so every
// 16-byte load of a wave covers 1 KB of contiguous weights.  Group t + 256 j
// lies in the block's 2048-weight tile j, so tile j's escapes are the
// code-15 weights of the threads' j-th groups, in thread order.
//
// The escape records of the tensor are in weight order: block b's first
// record is the number of escapes in blocks 0 .. b-1.  k_pack counts each
// block's escapes; k_scan turns the counts into those prefix sums; k_emit
// writes each block's records from there.  For every block with at most
// `stage_cap` escapes k_pack stages the records themselves in the workspace
// (in weight order: the symbols as u16, the positions as u32, and the
// block's four per-tile counts), so k_emit copies them to their place in
// whole lines and reads neither the codes nor the weights again.  A block
// with more escapes (a dense escape band), or any block when nothing is
// staged (wc_encode_noalloc), has its codes and the weights of its escapes
// read again.

constexpr uint32_t kDirectRecords = 256;  // blocks with more records write them through LDS

// Per-tile exclusive scans of the threads' group escape counts over the
// block (tile j = the threads' j-th groups, in thread order), two tiles per
// 32-bit word: a tile holds at most 2048 escapes, so the halves never carry.
// ex01/ex23: this thread's exclusive prefix in tiles 0/1 and 2/3; tot01 /
// tot23: the tiles' totals.  Contains a block barrier.
struct BlockEsc {
  uint32_t ex01, ex23, tot01, tot23;
  __device__ uint32_t ex(int j) const {
    return (j < 2 ? (j == 0 ? ex01 : ex01 >> 16) : (j == 2 ? ex23 : ex23 >> 16)) & 0xFFFFu;
  }
  __device__ uint32_t tile(int j) const {
    return (j < 2 ? (j == 0 ? tot01 : tot01 >> 16) : (j == 2 ? tot23 : tot23 >> 16)) & 0xFFFFu;
  }
  __device__ uint32_t total() const {
    return (tot01 & 0xFFFFu) + (tot01 >> 16) + (tot23 & 0xFFFFu) + (tot23 >> 16);
  }
  // first escape of tile j relative to the block's first
  __device__ uint32_t tile_base(int j) const {
    uint32_t s = 0;
    for (int q = 0; q < j; ++q) s += tile(q);
    return s;
  }
};

__device__ inline BlockEsc block_escape_scan(const uint32_t emask[4], uint32_t (*wtot)[kBlockThreads / kWave]) {
  constexpr int kWpb = kBlockThreads / kWave;
  const int lane = lane_id();
  const int wib = wave_in_block();
  const uint32_t p01 = (uint32_t)__popc(emask[0]) | ((uint32_t)__popc(emask[1]) << 16);
  const uint32_t p23 = (uint32_t)__popc(emask[2]) | ((uint32_t)__popc(emask[3]) << 16);
  const uint32_t i01 = wave_incl_scan_dpp(p01), i23 = wave_incl_scan_dpp(p23);
  if (lane == kWave - 1) {
    wtot[0][wib] = i01;
    wtot[1][wib] = i23;
  }
  __syncthreads();
  BlockEsc e{0, 0, 0, 0};
  uint32_t b01 = 0, b23 = 0;
#pragma unroll
  for (int q = 0; q < kWpb; ++q) {
    b01 += q < wib ? wtot[0][q] : 0u;
    b23 += q < wib ? wtot[1][q] : 0u;
    e.tot01 += wtot[0][q];
    e.tot23 += wtot[1][q];
  }
  e.ex01 = b01 + i01 - p01;
  e.ex23 = b23 + i23 - p23;
  return e;
}

struct PackArgs {
  const uint16_t* w;
  uint8_t* container;
  uint32_t* cnt;        // per-block escape counts
  uint16_t* tcnt;       // staged blocks: escape counts of the block's 4 tiles
  uint16_t* stage;      // stage_cap symbols per block
  uint32_t* stage_pos;  // stage_cap positions per block (full form)
  uint32_t stage_cap;
  uint64_t n;
  wc_header h;
};

template <int LAYOUT>
__global__ __launch_bounds__(kBlockThreads) void k_pack(PackArgs a) {
  constexpr int kGroups = kPackBlock / 8;                                  // 1024
  constexpr int kRawBytes = LAYOUT == WC_LAYOUT_K15 ? 7 * kGroups : 8 * kGroups;
  constexpr int kShift = LAYOUT == WC_LAYOUT_K15 ? 7 : 8;
  __shared__ uint8_t lut[512];
  __shared__ uint32_t wtot[2][kBlockThreads / kWave];
  __shared__ __attribute__((aligned(16))) uint32_t img_codes[kGroups];     // 4 KB
  __shared__ __attribute__((aligned(16))) uint32_t img_raw[kRawBytes / 4];  // 7 or 8 KB
  const int tid = threadIdx.x;
  const wc_header& h = a.h;
  const bool with_esc = h.n_esc != 0;
  for (int sidx = tid; sidx < 512; sidx += kBlockThreads) lut[sidx] = 15;
  for (int q = tid; q < kGroups; q += kBlockThreads) img_codes[q] = 0;
  if (LAYOUT == WC_LAYOUT_BYTESPLIT)  // (the K15 image is written whole below)
    for (int q = tid; q < kRawBytes / 4; q += kBlockThreads) img_raw[q] = 0;
  __syncthreads();
  if (tid < (int)h.n_dict) lut[h.dict[tid]] = (uint8_t)tid;
  __syncthreads();

  const uint64_t blk = blockIdx.x;
  const uint64_t w0 = blk * kPackBlock;  // first weight of the block
  // a full block (every block but possibly the last) loads its four groups at once
  const bool full = w0 + kPackBlock <= a.n;
  uint32_t wd[4][4];  // per group: weights 2i (low half) and 2i+1 (high half)
  if (full) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)(a.w + w0) + tid + kBlockThreads * j);
      wd[j][0] = v[0]; wd[j][1] = v[1]; wd[j][2] = v[2]; wd[j][3] = v[3];
    }
  }
  uint32_t emask[4];  // per group: bit i set when weight i has code 15
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = tid + kBlockThreads * j;  // group within the block
    const uint64_t gw = w0 + 8u * (uint64_t)g;
    emask[j] = 0;
    if (!full) {
      wd[j][0] = wd[j][1] = wd[j][2] = wd[j][3] = 0;
      const uint32_t valid = gw >= a.n ? 0u : a.n - gw >= 8 ? 8u : (uint32_t)(a.n - gw);
      if (valid == 8) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)(a.w + gw));
        wd[j][0] = v[0]; wd[j][1] = v[1]; wd[j][2] = v[2]; wd[j][3] = v[3];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = (uint32_t)(2 * i) < valid ? a.w[gw + 2 * i] : 0u;
          const uint32_t hi = (uint32_t)(2 * i + 1) < valid ? a.w[gw + 2 * i + 1] : 0u;
          wd[j][i] = lo | (hi << 16);
        }
      }
    }
    // (a group past n has no valid weights: zero codes and raw bytes)
    const uint32_t valid = gw >= a.n ? 0u : a.n - gw >= 8 ? 8u : (uint32_t)(a.n - gw);
    // codes: nibble i = code of weight i (even weight in the low nibble)
    uint32_t cd = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = (wd[j][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const uint32_t code = (uint32_t)i < valid ? lut[b >> kShift] : 0u;
      emask[j] |= (code == 15u ? 1u : 0u) << i;
      cd |= code << (4 * i);
    }
    img_codes[g] = cd;
    if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
      // low bytes of weights 0..3 and 4..7
      uint32_t r0 = __builtin_amdgcn_perm(wd[j][1], wd[j][0], 0x06040200u);
      uint32_t r1 = __builtin_amdgcn_perm(wd[j][3], wd[j][2], 0x06040200u);
      if (valid < 8) {
        const uint64_t keep = valid ? (~0ull >> (64 - 8 * valid)) : 0ull;
        r0 &= (uint32_t)keep;
        r1 &= (uint32_t)(keep >> 32);
      }
      img_raw[2 * g] = r0;
      img_raw[2 * g + 1] = r1;
    } else {
      // The group's 8 mantissas of 7 bits (56 bits, LSB first) go to byte
      // 7g of the image.  Eight consecutive groups (lanes 8s..8s+7) fill 56
      // bytes = 7 aligned u64 words; word k of them is bits [8k, 8k+64) of
      // the lane-k and lane-(k+1) values side by side, so lanes 0..6 of each
      // eight store one word each, with their right neighbour's value from a
      // row shift.  (Every lane reaches this point: no divergence.)
      uint64_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint64_t mi = (uint32_t)i < valid ? (wd[j][i >> 1] >> (16 * (i & 1))) & 0x7Fu : 0u;
        m |= mi << (7 * i);
      }
      const uint32_t nlo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)m, 0x101, 0xF, 0xF, false);  // row_shl:1
      const uint32_t nhi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(m >> 32), 0x101, 0xF, 0xF, false);
      const uint64_t nxt = (uint64_t)nlo | ((uint64_t)nhi << 32);
      const int l8 = tid & 7;
      if (l8 < 7) ((uint64_t*)img_raw)[7 * (g >> 3) + l8] = (m >> (8 * l8)) | (nxt << (56 - 8 * l8));
    }
  }

  if (with_esc) {
    // (the scan's barrier also orders the image writes above before the copies below)
    const BlockEsc be = block_escape_scan(emask, wtot);
    const uint32_t total = be.total();
    if (tid == 0) a.cnt[blk] = total;
    if (total != 0 && total <= a.stage_cap) {
      // the block's records, in weight order, and its tiles' counts
      uint16_t* st = a.stage + blk * a.stage_cap;
      uint32_t* sp = a.stage_pos + blk * a.stage_cap;
      const bool compact = (h.flags & WC_FLAG_COMPACT) != 0;
      if (tid < 4) a.tcnt[4u * blk + tid] = (uint16_t)be.tile(tid);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t m = emask[j];
        uint32_t o = be.tile_base(j) + be.ex(j);
        const uint64_t gw = w0 + 8u * (uint64_t)(tid + kBlockThreads * j);
        while (m) {
          const int i = __builtin_ctz(m);
          m &= m - 1u;
          if (!compact) sp[o] = (uint32_t)(gw + (uint64_t)i);
          st[o++] = (uint16_t)(((wd[j][i >> 1] >> (16 * (i & 1))) & 0xFFFFu) >> kShift);
        }
      }
    }
  } else {
    __syncthreads();  // the images are complete before they are copied out
  }

  // the block's stream images, up to each stream's padded end
  {
    const uint64_t cpad = pad16((a.n + 1u) / 2u);
    const uint64_t c0 = blk * (kGroups * 4u);
    const uint64_t cend = c0 + kGroups * 4u < cpad ? c0 + kGroups * 4u : cpad;
    u32x4* dst = (u32x4*)(a.container + h.off_codes + c0);
    const u32x4* srcv = (const u32x4*)img_codes;
    for (uint64_t q = tid; c0 + 16u * q < cend; q += kBlockThreads) dst[q] = srcv[q];
    const uint64_t rpad = pad16(raw_bytes(LAYOUT, a.n));
    const uint64_t r0 = blk * kRawBytes;
    const uint64_t rend = r0 + kRawBytes < rpad ? r0 + kRawBytes : rpad;
    u32x4* rdst = (u32x4*)(a.container + h.off_raw + r0);
    const u32x4* rsrc = (const u32x4*)img_raw;
    for (uint64_t q = tid; r0 + 16u * q < rend; q += kBlockThreads) rdst[q] = rsrc[q];
  }
  // header and the escape streams' zero gaps
  if (blk == 0) {
    if (tid < 32) ((uint32_t*)a.container)[tid] = ((const uint32_t*)&a.h)[tid];
    if (tid == 32) {
      const uint64_t pe = h.off_esc_pos + pos_bytes(h.flags, h.n_esc);
      for (uint64_t o = pe; o < h.off_esc_sym; ++o) a.container[o] = 0;
      const uint64_t se = h.off_esc_sym + sym_bytes(LAYOUT) * h.n_esc;
      for (uint64_t o = se; o < h.off_esc_idx; ++o) a.container[o] = 0;
      const uint64_t ie = h.off_esc_idx + 4u * index_entries(h.n, h.n_esc);
      for (uint64_t o = ie; o < h.total_bytes; ++o) a.container[o] = 0;
    }
  }
}

// ---- scan of block escape counts -------------------------------------------
// One workgroup of 1024 threads: chunks of 16384 counts, thread t taking 16
// consecutive counts of a chunk; a carry joins the chunks.  Also writes the
// escape index's closing entry (the escape count).

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 16;

__global__ __launch_bounds__(kScanThreads) void k_scan(const uint32_t* __restrict__ cnt,
                                                       uint32_t* __restrict__ off, uint64_t nblk,
                                                       uint32_t* __restrict__ close_entry,
                                                       uint32_t n_esc) {
  __shared__ uint32_t wtot[kScanThreads / kWave];
  __shared__ uint32_t sh_carry;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wib = tid / kWave;
  if (tid == 0) {
    sh_carry = 0;
    *close_entry = n_esc;
  }
  __syncthreads();
  for (uint64_t base = 0; base < nblk; base += (uint64_t)kScanThreads * kScanPer) {
    const uint64_t i0 = base + (uint64_t)tid * kScanPer;
    uint32_t v[kScanPer];
    if (i0 + kScanPer <= nblk) {
#pragma unroll
      for (int k = 0; k < kScanPer; k += 4) {
        const u32x4 q = *(const u32x4*)(cnt + i0 + k);
        v[k] = q[0]; v[k + 1] = q[1]; v[k + 2] = q[2]; v[k + 3] = q[3];
      }
    } else {
#pragma unroll
      for (int k = 0; k < kScanPer; ++k) v[k] = i0 + k < nblk ? cnt[i0 + k] : 0u;
    }
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) s += v[k];
    const uint32_t ex = wave_excl_scan_u32(s);
    if (lane == kWave - 1) wtot[wib] = ex + s;
    __syncthreads();
    uint32_t before = 0, chunk = 0;
    for (int q = 0; q < kScanThreads / kWave; ++q) {
      before += q < wib ? wtot[q] : 0u;
      chunk += wtot[q];
    }
    uint32_t run = sh_carry + before + ex;
    if (i0 + kScanPer <= nblk) {
#pragma unroll
      for (int k = 0; k < kScanPer; k += 4) {
        u32x4 q;
        q[0] = run; run += v[k];
        q[1] = run; run += v[k + 1];
        q[2] = run; run += v[k + 2];
        q[3] = run; run += v[k + 3];
        *(u32x4*)(off + i0 + k) = q;
      }
    } else {
      for (int k = 0; k < kScanPer; ++k) {
        if (i0 + k < nblk) off[i0 + k] = run;
        run += v[k];
      }
    }
    __syncthreads();  // every thread has read sh_carry and wtot
    if (tid == 0) sh_carry += chunk;
    __syncthreads();
  }
}

// ---- escape records ---------------------------------------------------------
// A workgroup covers `group` consecutive encode blocks (kEmitMax when the
// escapes are sparse, so the grid is small and each workgroup's loads are in
// flight together; 1 when they average more than a stage per block, so that
// the blocks of dense bands, which read their codes and weights again, each
// keep a workgroup of their own).  Thread t copies record t of each staged
// block, so a block's records go out as one run of lane-contiguous stores.

constexpr int kEmitMax = 8;

struct EmitArgs {
  const uint16_t* w;
  uint8_t* container;
  const uint32_t* cnt;
  const uint32_t* off;
  const uint16_t* tcnt;
  const uint16_t* stage;
  const uint32_t* stage_pos;
  uint32_t stage_cap;
  uint32_t group;  // encode blocks per workgroup, 1..kEmitMax
  uint32_t ahead;  // stage slots (per block) loaded before the counts arrive, <= stage_cap
  uint64_t nblk;
  uint64_t n;
  wc_header h;
};

// Block `blk`'s `cntb` records from `excl` on, and its index entries, when
// they were not staged: the block's codes and the weights of its escapes are
// read again.  Contains block barriers (call it block-uniformly).
template <int LAYOUT>
__device__ void emit_dense(const EmitArgs& a, uint64_t blk, uint32_t cntb, uint32_t excl,
                           uint32_t (*wtot)[kBlockThreads / kWave], uint32_t* st_pos,
                           uint16_t* st_sym) {
  constexpr int kShift = LAYOUT == WC_LAYOUT_K15 ? 7 : 8;
  const int tid = threadIdx.x;
  const wc_header& h = a.h;
  const uint64_t w0 = blk * kPackBlock;
  const uint64_t n_tiles = (a.n + kTile - 1) / kTile;
  uint32_t* const index = (uint32_t*)(a.container + h.off_esc_idx);
  uint32_t* pos = (uint32_t*)(a.container + h.off_esc_pos);
  uint8_t* sym = a.container + h.off_esc_sym;
  const bool compact = (h.flags & WC_FLAG_COMPACT) != 0;
  // the block's codes, in k_pack's group mapping; codes past n are 0
  const uint32_t* codes = (const uint32_t*)(a.container + h.off_codes) + w0 / 8;
  uint32_t emask[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t gw = w0 + 8u * (uint64_t)(tid + kBlockThreads * j);
    const uint32_t c = gw < a.n ? codes[tid + kBlockThreads * j] : 0u;
    emask[j] = group_esc_bits(c);
  }
  const BlockEsc be = block_escape_scan(emask, wtot);
  if (tid < 4 && 4u * blk + (uint64_t)tid < n_tiles) index[4u * blk + tid] = excl + be.tile_base(tid);
  // the escaped symbols, from the weights again
  uint32_t wd[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wd[j][0] = wd[j][1] = wd[j][2] = wd[j][3] = 0;
    if (!emask[j]) continue;
    const uint64_t gw = w0 + 8u * (uint64_t)(tid + kBlockThreads * j);
    if (gw + 8 <= a.n) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)(a.w + gw));
      wd[j][0] = v[0]; wd[j][1] = v[1]; wd[j][2] = v[2]; wd[j][3] = v[3];
    } else {
      for (int i = 0; gw + i < a.n; ++i) wd[j][i >> 1] |= (uint32_t)a.w[gw + i] << (16 * (i & 1));
    }
  }
  auto sym_at = [&](int j, int i) -> uint32_t {
    return ((wd[j][i >> 1] >> (16 * (i & 1))) & 0xFFFFu) >> kShift;
  };
  if (cntb <= kDirectRecords) {
    // few records: each thread stores its own
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t m = emask[j];
      if (!m) continue;
      uint32_t r = be.tile_base(j) + be.ex(j);  // rank in the block
      const uint64_t gw = w0 + 8u * (uint64_t)(tid + kBlockThreads * j);
      while (m) {
        const int i = __builtin_ctz(m);
        m &= m - 1u;
        const uint64_t o = (uint64_t)excl + r;
        if (o < h.n_esc) {
          if (!compact) pos[o] = (uint32_t)(gw + (uint64_t)i);  // the compact form keeps symbols only
          if (LAYOUT == WC_LAYOUT_K15)
            ((uint16_t*)sym)[o] = (uint16_t)sym_at(j, i);
          else
            sym[o] = (uint8_t)sym_at(j, i);
        }
        ++r;
      }
    }
  } else {
    // many: each tile's records go through LDS in order and out with
    // lane-contiguous stores
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t tc = be.tile(j);
      if (tc == 0) continue;  // block-uniform
      const uint32_t tb = be.tile_base(j);
      uint32_t m = emask[j];
      uint32_t o = be.ex(j);
      const uint64_t gw = w0 + 8u * (uint64_t)(tid + kBlockThreads * j);
      while (m) {
        const int i = __builtin_ctz(m);
        m &= m - 1u;
        st_pos[o] = (uint32_t)(gw + (uint64_t)i);
        st_sym[o] = (uint16_t)sym_at(j, i);
        ++o;
      }
      __syncthreads();
      for (uint32_t q = (uint32_t)tid; q < tc; q += kBlockThreads) {
        const uint64_t oo = (uint64_t)excl + tb + q;
        if (oo < h.n_esc) {
          if (!compact) pos[oo] = st_pos[q];
          if (LAYOUT == WC_LAYOUT_K15)
            ((uint16_t*)sym)[oo] = st_sym[q];
          else
            sym[oo] = (uint8_t)st_sym[q];
        }
      }
      __syncthreads();
    }
  }
}

template <int LAYOUT, int G>
__global__ __launch_bounds__(kBlockThreads) void k_emit(EmitArgs a) {
  static_assert(G >= 1 && G <= kEmitMax, "blocks per workgroup");
  constexpr int kGroups = kPackBlock / 8;
  static_assert(WC_STAGE_SYMBOLS <= kBlockThreads, "one staged record of a block per thread");
  __shared__ uint32_t wtot[2][kBlockThreads / kWave];
  // a dense tile's records: 8 KB of positions, 4 KB of symbols
  __shared__ __attribute__((aligned(16))) uint32_t st_pos[2 * kGroups];
  __shared__ __attribute__((aligned(16))) uint16_t st_sym[2 * kGroups];
  const int tid = threadIdx.x;
  const wc_header& h = a.h;
  const uint64_t n_tiles = (a.n + kTile - 1) / kTile;
  const uint64_t b0 = (uint64_t)blockIdx.x * G;
  const uint32_t nb = (uint32_t)(a.nblk - b0 < (uint64_t)G ? a.nblk - b0 : (uint64_t)G);
  uint32_t* const index = (uint32_t*)(a.container + h.off_esc_idx);
  uint32_t* pos = (uint32_t*)(a.container + h.off_esc_pos);
  uint8_t* sym = a.container + h.off_esc_sym;
  const bool compact = (h.flags & WC_FLAG_COMPACT) != 0;
  // Thread t takes record t of each block's stage.  Threads below `ahead`
  // issue their stage loads before any count is known (the stage holds
  // stage_cap records per block, so the loads stay inside it, and those past
  // a block's count are not used); the others load only records that exist,
  // once the counts are in.
  uint32_t rs[G], rp[G];
  const bool staging = a.stage_cap != 0;
  const bool early = (uint32_t)tid < a.ahead;
  auto load_stage = [&](int i) {
    const uint64_t e = (b0 + (uint64_t)i) * a.stage_cap + (uint64_t)tid;
    rs[i] = a.stage[e];
    if (!compact) rp[i] = a.stage_pos[e];
  };
#pragma unroll
  for (int i = 0; i < G; ++i) {
    rs[i] = rp[i] = 0;
    if (early && staging && (uint32_t)i < nb) load_stage(i);
  }
  // index entries of the blocks that are not dense: lane 4i + j takes tile j of block i
  uint32_t ix_cnt = 0, ix_off = 0;
  uint64_t ix_tc = 0;
  const bool ix = tid < 4 * (int)nb;
  const uint64_t ix_blk = b0 + (uint64_t)(tid >> 2);
  if (ix) {
    ix_cnt = a.cnt[ix_blk];
    ix_off = a.off[ix_blk];
    if (staging) ix_tc = *(const uint64_t*)(a.tcnt + 4u * ix_blk);
  }
  // the group's counts and first records (uniform); dense: the blocks whose
  // records were not staged
  uint32_t c[G], o[G];
  uint32_t dense = 0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    c[i] = (uint32_t)i < nb ? a.cnt[b0 + i] : 0u;
    o[i] = (uint32_t)i < nb ? a.off[b0 + i] : 0u;
    dense |= (c[i] <= a.stage_cap ? 0u : 1u) << i;
  }
  if (!early && staging) {
#pragma unroll
    for (int i = 0; i < G; ++i)
      if ((uint32_t)tid < c[i] && c[i] <= a.stage_cap) load_stage(i);
  }
  if (ix) {
    const int j = tid & 3;
    if (ix_cnt <= a.stage_cap && 4u * ix_blk + (uint64_t)j < n_tiles) {
      uint32_t base = 0;
      if (ix_cnt != 0)  // the tile counts were staged with the records
        for (int q = 0; q < j; ++q) base += (uint32_t)(ix_tc >> (16 * q)) & 0xFFFFu;
      index[4u * ix_blk + j] = ix_off + base;
    }
  }
  if (staging) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const uint64_t r = (uint64_t)o[i] + (uint64_t)tid;
      if ((uint32_t)tid < c[i] && c[i] <= a.stage_cap && r < h.n_esc) {
        if (!compact) pos[r] = rp[i];
        if (LAYOUT == WC_LAYOUT_K15)
          ((uint16_t*)sym)[r] = (uint16_t)rs[i];
        else
          sym[r] = (uint8_t)rs[i];
      }
    }
  }
  while (dense) {  // uniform
    const int i = __builtin_ctz(dense);
    dense &= dense - 1u;
    const uint64_t blk = b0 + (uint64_t)i;
    emit_dense<LAYOUT>(a, blk, a.cnt[blk], a.off[blk], wtot, st_pos, st_sym);
  }
}

// Encode with the block state at `state` (16-byte aligned: counts, offsets,
// then, when stage_cap > 0, per block 4 u16 tile counts, stage_cap u16
// symbols and stage_cap u32 positions).
static hipError_t launch_encode_state(const wc_header& h, const uint16_t* w, uint8_t* container,
                                      uint8_t* state, uint32_t stage_cap, hipStream_t s) {
  if (h.layout == WC_LAYOUT_RAW) return launch_encode_raw(h, w, container, s);
  const uint64_t nblk = (h.n + kPackBlock - 1) / kPackBlock;
  // counts and offsets each start 16-byte aligned (k_scan moves them 16 bytes at a time)
  const uint64_t nblk4 = (nblk + 3) & ~(uint64_t)3;
  uint32_t* cnt = (uint32_t*)state;
  uint32_t* off = cnt + nblk4;
  uint16_t* tcnt = stage_cap ? (uint16_t*)(state + 8u * nblk4) : nullptr;
  uint16_t* stage = stage_cap ? (uint16_t*)(state + 16u * nblk4) : nullptr;
  uint32_t* stage_pos =
      stage_cap ? (uint32_t*)(state + 16u * nblk4 + 2u * (uint64_t)stage_cap * nblk) : nullptr;
  PackArgs p;
  p.w = w;
  p.container = container;
  p.cnt = cnt;
  p.tcnt = tcnt;
  p.stage = stage;
  p.stage_pos = stage_pos;
  p.stage_cap = stage_cap;
  p.n = h.n;
  p.h = h;
  // n == 0 still runs one block: it writes the header
  const dim3 grid((unsigned)(nblk ? nblk : 1));
  if (h.layout == WC_LAYOUT_K15)
    hipLaunchKernelGGL(k_pack<WC_LAYOUT_K15>, grid, dim3(kBlockThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_pack<WC_LAYOUT_BYTESPLIT>, grid, dim3(kBlockThreads), 0, s, p);
  if (h.n_esc == 0 || nblk == 0) return hipGetLastError();
  const uint64_t n_tiles = (h.n + kTile - 1) / kTile;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, s, (const uint32_t*)cnt, off, nblk,
                     (uint32_t*)(container + h.off_esc_idx) + n_tiles, (uint32_t)h.n_esc);
  EmitArgs e;
  e.w = w;
  e.container = container;
  e.cnt = cnt;
  e.off = off;
  e.tcnt = tcnt;
  e.stage = stage;
  e.stage_pos = stage_pos;
  e.stage_cap = stage_cap;
  // kEmitMax blocks per workgroup, unless the escapes average more than a
  // stage per block (dense bands) or nothing is staged
  e.group = h.n_esc > (uint64_t)stage_cap * nblk ? 1u : (uint32_t)kEmitMax;
  // Stage slots loaded ahead of the counts: all of them when the blocks of
  // a sparse tensor average a quarter stage or more (6144x24576 N(0,0.015)
  // K15, 160 records per block: 14.1 -> 10.5 us), none when they average
  // less (byte-split there, 2 per block: 7.6 against 8.2 us with all); with
  // dense bands (one block per workgroup), whose other blocks hold few
  // records, the first 64 (all slots: 6144x24576 banded byte-split 45 ->
  // 56 us).
  e.ahead = e.group == 1u ? (stage_cap < 64u ? stage_cap : 64u)
            : 4u * h.n_esc >= (uint64_t)stage_cap * nblk ? stage_cap : 0u;
  e.nblk = nblk;
  e.n = h.n;
  e.h = h;
  const dim3 egrid((unsigned)((nblk + e.group - 1) / e.group));
  // (one block per workgroup has its own instance: the group's arrays would
  // take registers from the dense path and halve the waves per SIMD)
  if (h.layout == WC_LAYOUT_K15) {
    if (e.group == 1)
      hipLaunchKernelGGL((k_emit<WC_LAYOUT_K15, 1>), egrid, dim3(kBlockThreads), 0, s, e);
    else
      hipLaunchKernelGGL((k_emit<WC_LAYOUT_K15, kEmitMax>), egrid, dim3(kBlockThreads), 0, s, e);
  } else {
    if (e.group == 1)
      hipLaunchKernelGGL((k_emit<WC_LAYOUT_BYTESPLIT, 1>), egrid, dim3(kBlockThreads), 0, s, e);
    else
      hipLaunchKernelGGL((k_emit<WC_LAYOUT_BYTESPLIT, kEmitMax>), egrid, dim3(kBlockThreads), 0, s, e);
  }
  return hipGetLastError();
}

hipError_t launch_encode(const wc_header& h, const uint16_t* w, uint8_t* container, uint8_t* work,
                         hipStream_t s) {
  return launch_encode_state(h, w, container, work + kWorkBlocks, WC_STAGE_SYMBOLS, s);
}

// ---- encode without a workspace --------------------------------------------
// For callers that cannot allocate: the block counts and offsets live in a
// fixed device array of the library, one per GPU, held until the process
// ends, sized for the largest tensor taken (WC_NOALLOC_MAX_N weights, 8
// bytes per 8192-weight block).  Nothing is staged there, so k_emit reads
// the codes and weights of every block with escapes again; the container is
// the same.
// In host code the array's name stands for a host-side symbol, not a device
// address: its device address is looked up once per device and only that
// address reaches the kernels.  Every call rewrites the counts and offsets
// of its blocks before reading them, so nothing needs clearing.  Calls that
// overlap on one GPU share the array and race.
constexpr size_t kScratchBytes = 8u * (WC_NOALLOC_MAX_N / kPackBlock) + 32u;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[64];

static hipError_t scratch_address(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = (uint8_t*)g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_encode_noalloc(const wc_header& h, const uint16_t* w, uint8_t* container,
                                 hipStream_t s) {
  uint8_t* sp = nullptr;
  const hipError_t e = scratch_address(&sp);
  if (e != hipSuccess) return e;
  return launch_encode_state(h, w, container, sp, 0, s);
}

}  // namespace wc
