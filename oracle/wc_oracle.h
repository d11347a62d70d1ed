/*
 * wc_oracle.h — CPU oracle for lossless BF16 sign+exponent coding.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call this library.  The GPU library never
 * includes, links or calls it, and this file shares no code with the GPU
 * library: the container layout is parsed and written here by code of its
 * own.
 *
 * What it computes (sources, by page title and section):
 *  - BF16 = 1 sign bit, 8 exponent bits, 7 mantissa bits; trained weights
 *    reuse a narrow set of sign+exponent combinations, so frequent symbols
 *    get short codes and rare ones go to an exact escape stream:
 *    page "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está listo
 *    para producción?", section "¿Qué demostró realmente el experimento con
 *    GLM-5.2?".
 *  - K15 layout: the 9-bit sign+exponent symbol becomes a 4-bit code into a
 *    15-entry table, rare 9-bit symbols go to an exact escape stream, the 7-bit
 *    mantissa is kept uncompressed, and bits/weight count all overhead;
 *    byte-split layout: the high byte is rebuilt from a dictionary, code
 *    indices and an escape stream while the low byte is left unchanged:
 *    page "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%", section
 *    "Cómo funciona la compresión".
 *  - Lossless means every source bit is rebuilt; rebuilt weights may be used
 *    at once inside the matrix product; a changed accumulation order changes
 *    outputs even with exact weights: page "Compresión de pesos LLM sin
 *    pérdida vs 8-bit GGUF…", section "¿Qué significa “sin pérdida” para los
 *    pesos de un LLM?".
 *
 * Every function is a direct, unblocked, single-threaded loop.  Readings of
 * points the pages leave open are listed in the repository's design notes
 * and restated next to the code that takes them.
 */
#ifndef WC_ORACLE_H
#define WC_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_LAYOUT_BYTESPLIT 0
#define ORC_LAYOUT_K15 1
#define ORC_LAYOUT_RAW 2 /* the BF16 bit patterns stored as they are */

/* Container flags (header byte 104).  ORC_FLAG_COMPACT: the escape stream
 * holds the symbols only, in weight order; the k-th weight whose code is 15
 * takes the k-th symbol (no position stream).  Coded layouts only. */
#define ORC_FLAG_COMPACT 1

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_SIZE (-2)
#define ORC_E_CORRUPT (-3)

/* Symbol histogram: counts[s] for s < 256 (byte-split) or s < 512 (K15). */
int orc_histogram(int layout, const uint16_t *w, uint64_t n, uint64_t *counts);

/* Top-15 dictionary from a histogram.  dict[16] receives the symbols by rank
 * (unused slots and slot 15 are 0); *n_dict the number of entries; *n_esc the
 * number of weights whose symbol is not in the dictionary. */
int orc_dictionary(int layout, const uint64_t *counts, uint64_t n,
                   uint16_t dict[16], int *n_dict, uint64_t *n_esc);

/* Exact container size for n weights with n_esc escapes (flags 0, or
 * with the given flags). */
int orc_container_size(int layout, uint64_t n, uint64_t n_esc, uint64_t *total);
int orc_container_size_flags(int layout, int flags, uint64_t n, uint64_t n_esc,
                             uint64_t *total);

/* The layout whose container is smallest for w[0..n): byte-split, K15 or
 * raw, ties to the lower layout number. */
int orc_choose_layout(const uint16_t *w, uint64_t n, int *layout);

/* Full encode into out[0..cap); *size receives the container size
 * (orc_encode: flags 0). */
int orc_encode(int layout, const uint16_t *w, uint64_t n,
               uint8_t *out, uint64_t cap, uint64_t *size);
int orc_encode_flags(int layout, int flags, const uint16_t *w, uint64_t n,
                     uint8_t *out, uint64_t cap, uint64_t *size);

/* Header fields of a container (parsed by the oracle's own reader).
 * offsets: codes, raw, escape positions, escape symbols, total bytes,
 * escape index. */
int orc_header_info(const uint8_t *c, uint64_t size, int *layout, int *n_dict,
                    uint64_t *n, uint64_t *n_esc, uint16_t dict[16],
                    uint64_t offsets[6]);

/* The flags byte of a valid container. */
int orc_header_flags(const uint8_t *c, uint64_t size, int *flags);

/* Decode a container into out[0..n). */
int orc_decode(const uint8_t *c, uint64_t size, uint16_t *out, uint64_t n_cap);

/* y[b][r] = sum_c f32(W[r][c]) * f32(x[b][c]); fp32 products, fp32 sum in
 * ascending c. */
int orc_gemv_f32(const uint16_t *W, uint64_t rows, uint64_t cols,
                 const uint16_t *x, uint32_t batch, float *y);

/* Same sum in fp64; a[b][r] = sum_c |W[r][c] * x[b][c]| (fp64). */
int orc_gemv_f64(const uint16_t *W, uint64_t rows, uint64_t cols,
                 const uint16_t *x, uint32_t batch, double *y, double *a);

/* bits per weight = 8 * container bytes / n, and the payload part (streams
 * without header and padding). */
int orc_bits_per_weight(const uint8_t *c, uint64_t size, double *bpw,
                        double *payload_bpw);

#ifdef __cplusplus
}
#endif
#endif
