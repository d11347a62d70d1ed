/*
 * wc_oracle.c — plain CPU oracle for lossless BF16 sign+exponent coding,
 * its exact decode, the GEMV on the rebuilt weights and the bits/weight
 * accounting.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library, with which it
 * shares no code.
 *
 * Sources (page title, section):
 *  [P2] "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está listo
 *       para producción?" — sections "¿Qué significa “sin pérdida” para los
 *       pesos de un LLM?" and "¿Qué demostró realmente el experimento con
 *       GLM-5.2?".
 *  [P3] "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%" — section
 *       "Cómo funciona la compresión".
 *
 * The method is exact, so this oracle is the definition written out, one
 * weight at a time, in the order the pages describe: symbol + raw split,
 * symbol counts, a 15-entry dictionary of the most frequent symbols, one
 * 4-bit code per weight (code 15 = escape), the raw part stored unchanged,
 * rare symbols in an exact escape stream; decode rebuilds each weight from
 * the dictionary (or the escape stream) and its raw part.
 *
 * Readings where the pages are silent (each restated at its use):
 *  - byte-split symbol = high byte (b >> 8); K15 symbol = b >> 7 (9 bits);
 *  - dictionary = the min(15, #distinct) symbols of largest count, ties to
 *    the smaller symbol value; code = rank; code 15 marks an escape;
 *  - codes: two per byte, the even-index weight in the low nibble;
 *  - K15 mantissas: one LSB-first bitstream, mantissa i at bits [7i, 7i+7);
 *  - escape stream: ascending u32 positions, then the symbols (u8 for
 *    byte-split, u16 for K15), then (only when there are escapes) an index:
 *    for every multiple of 2048 weights j*2048 up to the tensor's last tile
 *    end, the number of escapes at positions below it (u32);
 *  - container: 128-byte little-endian header, then the five streams, each
 *    starting at a 16-byte aligned offset, gaps and tail zero;
 *  - raw layout (a BF16 fallback per tensor): no dictionary, codes or
 *    escapes, the weights as u16 in the raw stream; a tensor takes the
 *    layout (byte-split, K15 or raw) with the smallest container, ties to
 *    the lower layout number.
 */
#include "wc_oracle.h"

#include <string.h>

#define ORC_MAGIC 0x36314357u /* bytes "WC16" */
#define ORC_VERSION 2u
#define ORC_HEADER_BYTES 128u
#define ORC_INDEX_TILE 2048u /* weights per escape-index entry */
#define ORC_FLAGS_AT 104u     /* header byte holding the container flags */

/* ---- little-endian field access (byte by byte) ------------------------- */

static void put_le(uint8_t *p, uint64_t v, int bytes) {
  for (int k = 0; k < bytes; ++k) p[k] = (uint8_t)(v >> (8 * k));
}

static uint64_t get_le(const uint8_t *p, int bytes) {
  uint64_t v = 0;
  for (int k = 0; k < bytes; ++k) v |= (uint64_t)p[k] << (8 * k);
  return v;
}

static uint64_t pad16(uint64_t x) { return (x + 15u) / 16u * 16u; }

/* ---- the BF16 split [P2 "¿Qué demostró…"; P3 "Cómo funciona…"] ---------
 * Bits of a BF16 weight b: b[15] sign, b[14:7] exponent, b[6:0] mantissa.
 * Byte-split: symbol = high byte = sign + exponent[7:1]; raw = low byte =
 * exponent[0] + mantissa.  K15: symbol = sign + exponent (9 bits); raw =
 * the 7-bit mantissa. */

static int n_symbols(int layout) { return layout == ORC_LAYOUT_K15 ? 512 : 256; }
static int symbol_shift(int layout) { return layout == ORC_LAYOUT_K15 ? 7 : 8; }

static uint32_t symbol_of(int layout, uint16_t b) {
  return (uint32_t)b >> symbol_shift(layout);
}

static uint32_t raw_of(int layout, uint16_t b) {
  return (uint32_t)b & ((1u << symbol_shift(layout)) - 1u);
}

static uint64_t raw_stream_bytes(int layout, uint64_t n) {
  /* byte-split keeps one low byte per weight; K15 keeps 7 bits per weight;
   * raw keeps the whole 16-bit weight */
  if (layout == ORC_LAYOUT_RAW) return 2u * n;
  return layout == ORC_LAYOUT_K15 ? (7u * n + 7u) / 8u : n;
}

/* two 4-bit codes per byte; the raw layout has no codes */
static uint64_t code_stream_bytes(int layout, uint64_t n) {
  return layout == ORC_LAYOUT_RAW ? 0u : (n + 1u) / 2u;
}

static uint64_t sym_bytes(int layout) { return layout == ORC_LAYOUT_K15 ? 2u : 1u; }

/* escape-index entries: one per 2048-weight tile start plus the end, and
 * none at all without escapes */
static uint64_t index_entries(uint64_t n, uint64_t e) {
  return e ? (n + ORC_INDEX_TILE - 1u) / ORC_INDEX_TILE + 1u : 0u;
}

static int layout_ok(int layout) {
  return layout == ORC_LAYOUT_BYTESPLIT || layout == ORC_LAYOUT_K15 || layout == ORC_LAYOUT_RAW;
}

/* layouts with a dictionary and escapes */
static int coded(int layout) { return layout != ORC_LAYOUT_RAW; }

/* bytes of the escape-position stream: one u32 per escape, none in the
 * compact form, whose positions are implied by the code-15 marks */
static uint64_t pos_bytes(int flags, uint64_t e) {
  return (flags & ORC_FLAG_COMPACT) ? 0u : 4u * e;
}

/* stream offsets for n weights and e escapes, in the header's field order:
 * off[0] codes, off[1] raw, off[2] escape positions, off[3] escape symbols,
 * off[4] total container bytes, off[5] escape index (the last stream) */
static void layout_offsets(int layout, int flags, uint64_t n, uint64_t e, uint64_t off[6]) {
  off[0] = ORC_HEADER_BYTES;
  off[1] = pad16(off[0] + code_stream_bytes(layout, n));
  off[2] = pad16(off[1] + raw_stream_bytes(layout, n));
  off[3] = pad16(off[2] + pos_bytes(flags, e));
  off[5] = pad16(off[3] + sym_bytes(layout) * e);
  off[4] = pad16(off[5] + 4u * index_entries(n, e));
}

/* ---- step 1: symbol counts ------------------------------------------- */

int orc_histogram(int layout, const uint16_t *w, uint64_t n, uint64_t *counts) {
  if (!layout_ok(layout) || !coded(layout) || !counts || (n && !w)) return ORC_E_ARG;
  for (int s = 0; s < n_symbols(layout); ++s) counts[s] = 0;
  for (uint64_t i = 0; i < n; ++i) counts[symbol_of(layout, w[i])] += 1;
  return ORC_OK;
}

/* ---- step 2: the 15-entry dictionary [P3 "Cómo funciona…"] -----------
 * Frequent symbols get the short codes: repeatedly take the unpicked symbol
 * with the largest nonzero count (ties: smaller symbol value), at most 15
 * times.  Its rank is its code.  Code 15 is left for escapes. */

int orc_dictionary(int layout, const uint64_t *counts, uint64_t n,
                   uint16_t dict[16], int *n_dict, uint64_t *n_esc) {
  if (!layout_ok(layout) || !coded(layout) || !counts || !dict || !n_dict || !n_esc) return ORC_E_ARG;
  int picked[512];
  memset(picked, 0, sizeof picked);
  for (int k = 0; k < 16; ++k) dict[k] = 0;
  uint64_t covered = 0;
  int nd = 0;
  while (nd < 15) {
    int best = -1;
    for (int s = 0; s < n_symbols(layout); ++s) {
      if (picked[s] || counts[s] == 0) continue;
      if (best < 0 || counts[s] > counts[best]) best = s; /* '>' keeps the smaller symbol on ties */
    }
    if (best < 0) break;
    picked[best] = 1;
    dict[nd++] = (uint16_t)best;
    covered += counts[best];
  }
  *n_dict = nd;
  *n_esc = n - covered;
  return ORC_OK;
}

/* the flags a layout may carry: the compact escape form needs escapes'
 * codes, so the raw layout takes none */
static int flags_ok(int layout, int flags) {
  return flags == 0 || (flags == ORC_FLAG_COMPACT && coded(layout));
}

int orc_container_size_flags(int layout, int flags, uint64_t n, uint64_t n_esc,
                             uint64_t *total) {
  if (!layout_ok(layout) || !flags_ok(layout, flags) || !total) return ORC_E_ARG;
  if (n >= (1ull << 32)) return ORC_E_SIZE;
  if (n_esc > n || (!coded(layout) && n_esc)) return ORC_E_ARG;
  uint64_t off[6];
  layout_offsets(layout, flags, n, n_esc, off);
  *total = off[4];
  return ORC_OK;
}

int orc_container_size(int layout, uint64_t n, uint64_t n_esc, uint64_t *total) {
  return orc_container_size_flags(layout, 0, n, n_esc, total);
}

/* ---- layout choice [the pages ask for a BF16 fallback: page "Compresión
 * de pesos LLM sin pérdida vs 8-bit GGUF…", section "Preguntas para un
 * vendor o equipo de investigación"] --------------------------------------
 * Each layout's container size follows from its escape count; the smallest
 * wins, ties to the lower layout number. */

int orc_choose_layout(const uint16_t *w, uint64_t n, int *layout) {
  if (!layout || (n && !w)) return ORC_E_ARG;
  if (n >= (1ull << 32)) return ORC_E_SIZE;
  int best = -1;
  uint64_t best_total = 0;
  for (int lay = ORC_LAYOUT_BYTESPLIT; lay <= ORC_LAYOUT_RAW; ++lay) {
    uint64_t e = 0;
    if (coded(lay)) {
      uint64_t counts[512];
      uint16_t dict[16];
      int n_dict;
      orc_histogram(lay, w, n, counts);
      orc_dictionary(lay, counts, n, dict, &n_dict, &e);
    }
    uint64_t total;
    orc_container_size(lay, n, e, &total);
    if (best < 0 || total < best_total) {
      best = lay;
      best_total = total;
    }
  }
  *layout = best;
  return ORC_OK;
}

/* ---- steps 3–6: codes, raw stream, escape stream, container ----------- */

int orc_encode_flags(int layout, int flags, const uint16_t *w, uint64_t n,
                     uint8_t *out, uint64_t cap, uint64_t *size) {
  if (!layout_ok(layout) || !flags_ok(layout, flags) || !out || !size || (n && !w))
    return ORC_E_ARG;
  if (n >= (1ull << 32)) return ORC_E_SIZE; /* positions are u32 */

  if (!coded(layout)) {
    /* raw: header, then every weight as a little-endian u16 */
    uint64_t off[6];
    layout_offsets(layout, 0, n, 0, off);
    if (cap < off[4]) return ORC_E_SIZE;
    memset(out, 0, off[4]);
    for (uint64_t i = 0; i < n; ++i) put_le(out + off[1] + 2u * i, w[i], 2);
    put_le(out + 0, ORC_MAGIC, 4);
    put_le(out + 4, ORC_VERSION, 2);
    put_le(out + 6, (uint64_t)layout, 1);
    put_le(out + 8, n, 8);
    for (int k = 0; k < 6; ++k) put_le(out + 56 + 8 * k, off[k], 8);
    *size = off[4];
    return ORC_OK;
  }

  uint64_t counts[512];
  orc_histogram(layout, w, n, counts);
  uint16_t dict[16];
  int n_dict;
  uint64_t n_esc;
  orc_dictionary(layout, counts, n, dict, &n_dict, &n_esc);

  uint64_t off[6];
  layout_offsets(layout, flags, n, n_esc, off);
  if (cap < off[4]) return ORC_E_SIZE;
  memset(out, 0, off[4]); /* gaps and tails are zero */

  /* symbol -> code: the rank in the dictionary, or 15 (escape) */
  uint8_t code_of[512];
  for (int s = 0; s < 512; ++s) code_of[s] = 15;
  for (int k = 0; k < n_dict; ++k) code_of[dict[k]] = (uint8_t)k;

  uint8_t *codes = out + off[0];
  uint8_t *raw = out + off[1];
  uint8_t *esc_pos = out + off[2];
  uint8_t *esc_sym = out + off[3];
  uint8_t *esc_idx = out + off[5];
  uint64_t e = 0;
  for (uint64_t i = 0; i < n; ++i) {
    /* index entry of each tile: the escapes seen before its first weight */
    if (n_esc && i % ORC_INDEX_TILE == 0) put_le(esc_idx + 4u * (i / ORC_INDEX_TILE), e, 4);
    uint32_t s = symbol_of(layout, w[i]);
    uint32_t r = raw_of(layout, w[i]);
    uint32_t c = code_of[s];
    /* 4-bit code: weight i sits in byte i/2, low nibble when i is even */
    codes[i / 2] |= (uint8_t)(c << ((i % 2) * 4));
    /* raw part stored unchanged */
    if (layout == ORC_LAYOUT_BYTESPLIT) {
      raw[i] = (uint8_t)r;
    } else {
      for (int k = 0; k < 7; ++k) {
        uint64_t bit = 7u * i + (uint64_t)k;
        raw[bit / 8] |= (uint8_t)(((r >> k) & 1u) << (bit % 8));
      }
    }
    /* rare symbol: exact escape record (position, symbol) in weight order;
     * the compact form keeps the symbol only (its position is the weight's
     * code-15 mark) */
    if (c == 15) {
      if (!(flags & ORC_FLAG_COMPACT)) put_le(esc_pos + 4u * e, i, 4);
      put_le(esc_sym + sym_bytes(layout) * e, s, (int)sym_bytes(layout));
      e += 1;
    }
  }

  /* the closing entry: every escape lies below the last tile's end */
  if (n_esc) put_le(esc_idx + 4u * (index_entries(n, n_esc) - 1u), e, 4);

  uint8_t *h = out;
  put_le(h + 0, ORC_MAGIC, 4);
  put_le(h + 4, ORC_VERSION, 2);
  put_le(h + 6, (uint64_t)layout, 1);
  put_le(h + 7, (uint64_t)n_dict, 1);
  put_le(h + 8, n, 8);
  put_le(h + 16, n_esc, 8);
  for (int k = 0; k < 16; ++k) put_le(h + 24 + 2 * k, dict[k], 2);
  for (int k = 0; k < 6; ++k) put_le(h + 56 + 8 * k, off[k], 8);
  put_le(h + ORC_FLAGS_AT, (uint64_t)flags, 1);
  *size = off[4];
  return ORC_OK;
}

int orc_encode(int layout, const uint16_t *w, uint64_t n,
               uint8_t *out, uint64_t cap, uint64_t *size) {
  return orc_encode_flags(layout, 0, w, n, out, cap, size);
}

/* ---- header reader: every field checked against the definition -------- */

int orc_header_info(const uint8_t *c, uint64_t size, int *layout, int *n_dict,
                    uint64_t *n, uint64_t *n_esc, uint16_t dict[16],
                    uint64_t offsets[6]) {
  if (!c || !layout || !n_dict || !n || !n_esc || !dict || !offsets) return ORC_E_ARG;
  if (size < ORC_HEADER_BYTES) return ORC_E_CORRUPT;
  if (get_le(c + 0, 4) != ORC_MAGIC || get_le(c + 4, 2) != ORC_VERSION) return ORC_E_CORRUPT;
  int lay = (int)c[6];
  int nd = (int)c[7];
  if (!layout_ok(lay) || nd > 15) return ORC_E_CORRUPT;
  uint64_t nn = get_le(c + 8, 8), ne = get_le(c + 16, 8);
  if (nn >= (1ull << 32) || ne > nn) return ORC_E_CORRUPT;
  if (!coded(lay) && (nd != 0 || ne != 0)) return ORC_E_CORRUPT;
  for (int k = 0; k < 16; ++k) {
    dict[k] = (uint16_t)get_le(c + 24 + 2 * k, 2);
    if (k >= nd && dict[k] != 0) return ORC_E_CORRUPT;
    if (k < nd && dict[k] >= n_symbols(lay)) return ORC_E_CORRUPT;
    for (int j = 0; j < k && k < nd; ++j)
      if (dict[j] == dict[k]) return ORC_E_CORRUPT;
  }
  int fl = (int)c[ORC_FLAGS_AT];
  if (!flags_ok(lay, fl)) return ORC_E_CORRUPT;
  uint64_t want[6];
  layout_offsets(lay, fl, nn, ne, want);
  for (int k = 0; k < 6; ++k) {
    offsets[k] = get_le(c + 56 + 8 * k, 8);
    if (offsets[k] != want[k]) return ORC_E_CORRUPT;
  }
  for (int k = ORC_FLAGS_AT + 1; k < 128; ++k)
    if (c[k] != 0) return ORC_E_CORRUPT;
  if (offsets[4] > size) return ORC_E_CORRUPT;
  *layout = lay;
  *n_dict = nd;
  *n = nn;
  *n_esc = ne;
  return ORC_OK;
}

int orc_header_flags(const uint8_t *c, uint64_t size, int *flags) {
  int layout, n_dict;
  uint64_t n, n_esc, off[6];
  uint16_t dict[16];
  if (!flags) return ORC_E_ARG;
  int st = orc_header_info(c, size, &layout, &n_dict, &n, &n_esc, dict, off);
  if (st != ORC_OK) return st;
  *flags = (int)c[ORC_FLAGS_AT];
  return ORC_OK;
}

/* ---- decode [P3 "Cómo funciona…": high byte / 9-bit symbol rebuilt from
 * the dictionary, the codes and the escape stream; raw part unchanged] ---
 * Walks the weights in order with a cursor into the escape stream (a merge,
 * not a search); every escape record must sit at the weight it is used for. */

int orc_decode(const uint8_t *c, uint64_t size, uint16_t *out, uint64_t n_cap) {
  int layout, n_dict;
  uint64_t n, n_esc, off[6];
  uint16_t dict[16];
  int st = orc_header_info(c, size, &layout, &n_dict, &n, &n_esc, dict, off);
  if (st != ORC_OK) return st;
  if (n > n_cap || (n && !out)) return ORC_E_ARG;
  if (!coded(layout)) {
    for (uint64_t i = 0; i < n; ++i) out[i] = (uint16_t)get_le(c + off[1] + 2u * i, 2);
    return ORC_OK;
  }
  const uint8_t *codes = c + off[0];
  const uint8_t *raw = c + off[1];
  const uint8_t *esc_pos = c + off[2];
  const uint8_t *esc_sym = c + off[3];
  const uint8_t *esc_idx = c + off[5];
  const int compact = (c[ORC_FLAGS_AT] & ORC_FLAG_COMPACT) != 0;
  uint64_t e = 0;
  for (uint64_t i = 0; i < n; ++i) {
    /* every index entry must count the escapes before its tile */
    if (n_esc && i % ORC_INDEX_TILE == 0 && get_le(esc_idx + 4u * (i / ORC_INDEX_TILE), 4) != e)
      return ORC_E_CORRUPT;
    uint32_t code = (codes[i / 2] >> ((i % 2) * 4)) & 15u;
    uint32_t s;
    if (code == 15) {
      /* the e-th escape record belongs to the e-th code-15 weight; a full
       * record also names that weight's position */
      if (e >= n_esc || (!compact && get_le(esc_pos + 4u * e, 4) != i)) return ORC_E_CORRUPT;
      s = (uint32_t)get_le(esc_sym + sym_bytes(layout) * e, (int)sym_bytes(layout));
      if (s >= (uint32_t)n_symbols(layout)) return ORC_E_CORRUPT;
      e += 1;
    } else {
      if ((int)code >= n_dict) return ORC_E_CORRUPT;
      s = dict[code];
    }
    uint32_t r;
    if (layout == ORC_LAYOUT_BYTESPLIT) {
      r = raw[i];
    } else {
      r = 0;
      for (int k = 0; k < 7; ++k) {
        uint64_t bit = 7u * i + (uint64_t)k;
        r |= (uint32_t)((raw[bit / 8] >> (bit % 8)) & 1u) << k;
      }
    }
    out[i] = (uint16_t)((s << symbol_shift(layout)) | r);
  }
  if (e != n_esc) return ORC_E_CORRUPT;
  if (n_esc && get_le(esc_idx + 4u * (index_entries(n, n_esc) - 1u), 4) != e) return ORC_E_CORRUPT;
  return ORC_OK;
}

/* ---- GEMV on the exact weights [P2 "¿Qué significa “sin pérdida”…":
 * rebuilt weights are consumed at once by the matrix product; exact weights
 * do not fix the accumulation order] -------------------------------------
 * W is row-major [rows][cols]; x is [batch][cols]; y is [batch][rows].
 * A BF16 value is the upper half of an fp32 with a zero lower half. */

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

int orc_gemv_f32(const uint16_t *W, uint64_t rows, uint64_t cols,
                 const uint16_t *x, uint32_t batch, float *y) {
  if ((rows && cols && (!W || !x)) || (rows && batch && !y)) return ORC_E_ARG;
  for (uint32_t b = 0; b < batch; ++b) {
    for (uint64_t r = 0; r < rows; ++r) {
      float acc = 0.0f;
      for (uint64_t c = 0; c < cols; ++c) {
        float p = bf16_to_f32(W[r * cols + c]) * bf16_to_f32(x[(uint64_t)b * cols + c]);
        acc = acc + p;
      }
      y[(uint64_t)b * rows + r] = acc;
    }
  }
  return ORC_OK;
}

int orc_gemv_f64(const uint16_t *W, uint64_t rows, uint64_t cols,
                 const uint16_t *x, uint32_t batch, double *y, double *a) {
  if ((rows && cols && (!W || !x)) || (rows && batch && (!y || !a))) return ORC_E_ARG;
  for (uint32_t b = 0; b < batch; ++b) {
    for (uint64_t r = 0; r < rows; ++r) {
      double acc = 0.0, mag = 0.0;
      for (uint64_t c = 0; c < cols; ++c) {
        double p = (double)bf16_to_f32(W[r * cols + c]) *
                   (double)bf16_to_f32(x[(uint64_t)b * cols + c]);
        acc += p;
        mag += p < 0 ? -p : p;
      }
      y[(uint64_t)b * rows + r] = acc;
      a[(uint64_t)b * rows + r] = mag;
    }
  }
  return ORC_OK;
}

/* ---- accounting [P3 "Cómo funciona…": bits per weight with all overhead
 * included] -------------------------------------------------------------
 * bpw counts every container byte (header, dictionary, streams, padding);
 * payload_bpw counts the streams' own bytes only (the escape index is part
 * of the escape overhead). */

int orc_bits_per_weight(const uint8_t *c, uint64_t size, double *bpw,
                        double *payload_bpw) {
  int layout, n_dict;
  uint64_t n, n_esc, off[6];
  uint16_t dict[16];
  int st = orc_header_info(c, size, &layout, &n_dict, &n, &n_esc, dict, off);
  if (st != ORC_OK) return st;
  if (!bpw || !payload_bpw || n == 0) return ORC_E_ARG;
  uint64_t payload = code_stream_bytes(layout, n) + raw_stream_bytes(layout, n) +
                     pos_bytes(c[ORC_FLAGS_AT], n_esc) + sym_bytes(layout) * n_esc +
                     4u * index_entries(n, n_esc);
  *bpw = 8.0 * (double)off[4] / (double)n;
  *payload_bpw = 8.0 * (double)payload / (double)n;
  return ORC_OK;
}
