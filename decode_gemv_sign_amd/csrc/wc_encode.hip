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
//   encode:     k_pack (codes, raw stream, per-block escape counts, header and
//               zero gaps) -> k_scan (exclusive scan of the block counts) ->
//               k_emit (escape positions and symbols in weight order, and the
//               escape index: the records before each 2048-weight tile).
// Every output byte is a pure function of the input, so the container is
// byte-identical from run to run.
#include "wc_launch.h"

namespace wc {

// ---- histogram -----------------------------------------------------------

constexpr int kHistCopies = 16;   // replicated sub-histograms per workgroup
constexpr int kHistStride = 513;  // odd stride: copies of a bin sit in different LDS banks

__global__ void k_zero_hist(uint32_t* hist) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < 512 * kHistGlobal) hist[i] = 0;
}

__global__ __launch_bounds__(kBlockThreads) void k_hist(const uint16_t* __restrict__ w, uint64_t n,
                                                        uint32_t* __restrict__ hist) {
  __shared__ uint32_t sub[kHistCopies * kHistStride];
  for (int i = threadIdx.x; i < kHistCopies * kHistStride; i += kBlockThreads) sub[i] = 0;
  __syncthreads();
  // lanes spread over the copies, so the few very frequent symbols of a
  // skewed tensor do not serialise on one LDS address
  uint32_t* mine = sub + (lane_id() & (kHistCopies - 1)) * kHistStride;
  const uint64_t stride = (uint64_t)gridDim.x * kBlockThreads;
  const uint64_t gid = (uint64_t)blockIdx.x * kBlockThreads + threadIdx.x;
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
  for (int b = threadIdx.x; b < 512; b += kBlockThreads) {
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
  uint64_t blocks = (nvec + kBlockThreads - 1) / kBlockThreads;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_hist, dim3((unsigned)blocks), dim3(kBlockThreads), 0, s, w, n, hist);
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

// ---- pack ----------------------------------------------------------------

struct PackArgs {
  const uint16_t* w;
  uint8_t* container;
  uint32_t* blk_cnt;
  uint64_t n;
  wc_header h;
};

// Block b encodes weights [8192 b, 8192 b + 8192): 1024 groups of 8, thread t
// taking groups t, t+256, t+512, t+768, so every 16-byte input load of a wave
// covers 1 KB of contiguous weights.  The block's code and raw bytes are
// assembled in a zero-filled LDS image (K15 groups are 7 bytes, unaligned)
// and written out with aligned 16-byte stores up to each stream's padded end,
// which also writes the streams' zero padding.
template <int LAYOUT>
__global__ __launch_bounds__(kBlockThreads) void k_pack(PackArgs a) {
  constexpr int kGroups = kPackBlock / 8;                                  // 1024
  constexpr int kRawBytes = LAYOUT == WC_LAYOUT_K15 ? 7 * kGroups : 8 * kGroups;
  __shared__ uint8_t lut[512];
  __shared__ uint32_t wsum[kBlockThreads / kWave];
  __shared__ __attribute__((aligned(16))) uint32_t img_codes[kGroups];     // 4 KB
  __shared__ __attribute__((aligned(16))) uint32_t img_raw[kRawBytes / 4];  // 7 or 8 KB
  const int tid = threadIdx.x;
  for (int sidx = tid; sidx < 512; sidx += kBlockThreads) lut[sidx] = 15;
  for (int q = tid; q < kGroups; q += kBlockThreads) img_codes[q] = 0;
  for (int q = tid; q < kRawBytes / 4; q += kBlockThreads) img_raw[q] = 0;
  __syncthreads();
  if (tid < (int)a.h.n_dict) lut[a.h.dict[tid]] = (uint8_t)tid;
  __syncthreads();

  const wc_header& h = a.h;
  const uint64_t w0 = (uint64_t)blockIdx.x * kPackBlock;  // first weight of the block
  uint32_t esc = 0;
  uint8_t* rimg = (uint8_t*)img_raw;
  // a full block (every block but possibly the last) loads its four groups at once
  const bool full = w0 + kPackBlock <= a.n;
  u32x4 pre[4];
  if (full) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pre[j] = __builtin_nontemporal_load((const u32x4*)(a.w + w0) + tid + kBlockThreads * j);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = tid + kBlockThreads * j;  // group within the block
    const uint64_t gw = w0 + 8u * (uint64_t)g;
    if (gw >= a.n) continue;
    const uint32_t valid = a.n - gw >= 8 ? 8u : (uint32_t)(a.n - gw);
    uint32_t wd[4];  // weights 2i (low half) and 2i+1 (high half)
    if (full) {
      wd[0] = pre[j][0]; wd[1] = pre[j][1]; wd[2] = pre[j][2]; wd[3] = pre[j][3];
    } else if (valid == 8) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)(a.w + gw));
      wd[0] = v[0]; wd[1] = v[1]; wd[2] = v[2]; wd[3] = v[3];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (uint32_t)(2 * i) < valid ? a.w[gw + 2 * i] : 0u;
        const uint32_t hi = (uint32_t)(2 * i + 1) < valid ? a.w[gw + 2 * i + 1] : 0u;
        wd[i] = lo | (hi << 16);
      }
    }
    // codes: nibble i = code of weight i (even weight in the low nibble)
    uint32_t cd = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = (wd[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const uint32_t code = (uint32_t)i < valid ? lut[b >> (LAYOUT == WC_LAYOUT_K15 ? 7 : 8)] : 0u;
      esc += code == 15u ? 1u : 0u;
      cd |= code << (4 * i);
    }
    img_codes[g] = cd;
    if (LAYOUT == WC_LAYOUT_BYTESPLIT) {
      // low bytes of weights 0..3 and 4..7
      uint32_t r0 = __builtin_amdgcn_perm(wd[1], wd[0], 0x06040200u);
      uint32_t r1 = __builtin_amdgcn_perm(wd[3], wd[2], 0x06040200u);
      if (valid < 8) {
        const uint64_t keep = valid ? (~0ull >> (64 - 8 * valid)) : 0ull;
        r0 &= (uint32_t)keep;
        r1 &= (uint32_t)(keep >> 32);
      }
      img_raw[2 * g] = r0;
      img_raw[2 * g + 1] = r1;
    } else {
      // 8 mantissas of 7 bits = 56 bits, LSB first, at byte 7g of the image
      uint64_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint64_t mi = (uint32_t)i < valid ? (wd[i >> 1] >> (16 * (i & 1))) & 0x7Fu : 0u;
        m |= mi << (7 * i);
      }
#pragma unroll
      for (int k = 0; k < 7; ++k) rimg[7 * g + k] = (uint8_t)(m >> (8 * k));
    }
  }
  // escape count of the block
  const uint32_t ws = wave_sum_u32(esc);
  if (lane_id() == 0) wsum[tid / kWave] = ws;
  __syncthreads();
  if (tid == 0 && w0 < a.n) {  // n == 0 has no blocks to count
    uint32_t t = 0;
    for (int q = 0; q < kBlockThreads / kWave; ++q) t += wsum[q];
    a.blk_cnt[blockIdx.x] = t;
  }
  // the block's stream images, up to each stream's padded end
  {
    const uint64_t cpad = pad16((a.n + 1u) / 2u);
    const uint64_t c0 = (uint64_t)blockIdx.x * (kGroups * 4u);
    const uint64_t cend = c0 + kGroups * 4u < cpad ? c0 + kGroups * 4u : cpad;
    u32x4* dst = (u32x4*)(a.container + h.off_codes + c0);
    const u32x4* srcv = (const u32x4*)img_codes;
    for (uint64_t q = tid; c0 + 16u * q < cend; q += kBlockThreads) dst[q] = srcv[q];
    const uint64_t rpad = pad16(raw_bytes(LAYOUT, a.n));
    const uint64_t r0 = (uint64_t)blockIdx.x * kRawBytes;
    const uint64_t rend = r0 + kRawBytes < rpad ? r0 + kRawBytes : rpad;
    u32x4* rdst = (u32x4*)(a.container + h.off_raw + r0);
    const u32x4* rsrc = (const u32x4*)img_raw;
    for (uint64_t q = tid; r0 + 16u * q < rend; q += kBlockThreads) rdst[q] = rsrc[q];
  }
  // header and the escape streams' zero gaps
  if (blockIdx.x == 0) {
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

// ---- scan of block escape counts ----------------------------------------

__global__ __launch_bounds__(1024) void k_scan(const uint32_t* __restrict__ cnt,
                                               uint32_t* __restrict__ off, uint64_t nblk) {
  __shared__ uint32_t wtot[1024 / kWave];
  const uint64_t tid = threadIdx.x;
  const uint64_t seg = (nblk + 1023) / 1024;
  const uint64_t b0 = tid * seg;
  const uint64_t b1 = b0 + seg < nblk ? b0 + seg : nblk;
  uint32_t s = 0;
  for (uint64_t i = b0; i < b1; ++i) s += cnt[i];
  const uint32_t ex = wave_excl_scan_u32(s);
  if (lane_id() == kWave - 1) wtot[tid / kWave] = ex + s;
  __syncthreads();
  uint32_t wbase = 0;
  for (uint64_t q = 0; q < tid / kWave; ++q) wbase += wtot[q];
  uint32_t run = wbase + ex;
  for (uint64_t i = b0; i < b1; ++i) {
    off[i] = run;
    run += cnt[i];
  }
}

// ---- escape records --------------------------------------------------------

struct EmitArgs {
  const uint16_t* w;
  uint8_t* container;
  const uint32_t* blk_cnt;
  const uint32_t* blk_off;
  uint64_t n;
  wc_header h;
};

// Block b covers weights [8192 b, 8192 b + 8192): wave q of it covers exactly
// the 2048-weight tile 4 b + q, so the wave's first record number is that
// tile's escape-index entry.
template <int LAYOUT>
__global__ __launch_bounds__(kBlockThreads) void k_emit(EmitArgs a) {
  static_assert(kTile == (int)WC_INDEX_TILE && kPackBlock == 4 * kTile, "one index tile per wave");
  __shared__ uint32_t wtot[kBlockThreads / kWave];
  const int tid = threadIdx.x;
  uint32_t* const index = (uint32_t*)(a.container + a.h.off_esc_idx);
  const uint64_t n_tiles = (a.n + kTile - 1) / kTile;
  const uint64_t my_tile = (uint64_t)blockIdx.x * (kBlockThreads / kWave) + (uint64_t)(tid / kWave);
  if (blockIdx.x == gridDim.x - 1 && tid == 0) index[n_tiles] = (uint32_t)a.h.n_esc;  // closing entry
  if (a.blk_cnt[blockIdx.x] == 0) {  // whole block: no escapes
    if ((tid & (kWave - 1)) == 0 && my_tile < n_tiles) index[my_tile] = a.blk_off[blockIdx.x];
    return;
  }
  const uint64_t chunk = (uint64_t)blockIdx.x * kBlockThreads + (uint64_t)tid;
  const uint64_t base = chunk * kChunk;
  uint32_t mask = 0;  // bit i: weight base+i escapes
  if (base < a.n) {
    const uint32_t valid = a.n - base >= kChunk ? kChunk : (uint32_t)(a.n - base);
    const u32x4 c = *(const u32x4*)(a.container + a.h.off_codes + 16u * chunk);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const uint32_t code = (c[i >> 3] >> (4 * (i & 7))) & 15u;
      if (code == 15u && (uint32_t)i < valid) mask |= 1u << i;
    }
  }
  const uint32_t cnt = __popc(mask);
  const uint32_t ex = wave_excl_scan_u32(cnt);
  if (lane_id() == kWave - 1) wtot[tid / kWave] = ex + cnt;
  __syncthreads();
  uint32_t wbase = 0;
  for (int q = 0; q < tid / kWave; ++q) wbase += wtot[q];
  uint64_t o = (uint64_t)a.blk_off[blockIdx.x] + wbase + ex;
  if (lane_id() == 0 && my_tile < n_tiles) index[my_tile] = (uint32_t)o;  // ex == 0 in lane 0
  uint32_t* pos = (uint32_t*)(a.container + a.h.off_esc_pos);
  uint8_t* sym = a.container + a.h.off_esc_sym;
  const bool compact = (a.h.flags & WC_FLAG_COMPACT) != 0;
  while (mask) {
    const int i = __builtin_ctz(mask);
    mask &= mask - 1u;
    if (o < a.h.n_esc) {
      const uint64_t p = base + (uint64_t)i;
      const uint32_t s = (uint32_t)a.w[p] >> (LAYOUT == WC_LAYOUT_K15 ? 7 : 8);
      if (!compact) pos[o] = (uint32_t)p;  // the compact form keeps symbols only
      if (LAYOUT == WC_LAYOUT_K15)
        ((uint16_t*)sym)[o] = (uint16_t)s;
      else
        sym[o] = (uint8_t)s;
    }
    ++o;
  }
}

hipError_t launch_encode(const wc_header& h, const uint16_t* w, uint8_t* container, uint8_t* work,
                         hipStream_t s) {
  if (h.layout == WC_LAYOUT_RAW) return launch_encode_raw(h, w, container, s);
  const uint64_t nblk = (h.n + kPackBlock - 1) / kPackBlock;
  uint32_t* blk_cnt = (uint32_t*)(work + kWorkBlocks);
  uint32_t* blk_off = blk_cnt + nblk;
  PackArgs p;
  p.w = w;
  p.container = container;
  p.blk_cnt = blk_cnt;
  p.n = h.n;
  p.h = h;
  // n == 0 still runs one block: it writes the header
  const dim3 grid((unsigned)(nblk ? nblk : 1));
  if (h.layout == WC_LAYOUT_K15)
    hipLaunchKernelGGL(k_pack<WC_LAYOUT_K15>, grid, dim3(kBlockThreads), 0, s, p);
  else
    hipLaunchKernelGGL(k_pack<WC_LAYOUT_BYTESPLIT>, grid, dim3(kBlockThreads), 0, s, p);
  if (h.n_esc == 0 || nblk == 0) return hipGetLastError();
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, blk_cnt, blk_off, nblk);
  EmitArgs e;
  e.w = w;
  e.container = container;
  e.blk_cnt = blk_cnt;
  e.blk_off = blk_off;
  e.n = h.n;
  e.h = h;
  if (h.layout == WC_LAYOUT_K15)
    hipLaunchKernelGGL(k_emit<WC_LAYOUT_K15>, dim3((unsigned)nblk), dim3(kBlockThreads), 0, s, e);
  else
    hipLaunchKernelGGL(k_emit<WC_LAYOUT_BYTESPLIT>, dim3((unsigned)nblk), dim3(kBlockThreads), 0, s, e);
  return hipGetLastError();
}

}  // namespace wc
