/* oracle_check.c — drives the CPU oracle (oracle/wc_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer; test infrastructure,
 * built and run by tests/test_sanitizers.py.
 *
 * It exercises every entry point of the oracle on seeded inputs of the
 * shapes the parity tests use, round-trips every layout and escape form,
 * and feeds the decoder damaged containers: each byte of small containers
 * with one bit flipped, truncated buffers and headers of random bytes.  The
 * decoder must answer ORC_OK or ORC_E_CORRUPT and never touch memory outside
 * its buffers; the sanitizers turn any such access into a failed run.
 * Prints one line per group and exits 0 when every check held. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "wc_oracle.h"

static int failures = 0;

#define CHECK(cond, ...)                           \
  do {                                             \
    if (!(cond)) {                                 \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                \
      fputc('\n', stderr);                         \
      ++failures;                                  \
    }                                              \
  } while (0)

/* splitmix64: the seeded bit source of the inputs (no part of the method) */
static uint64_t mix_state;
static uint64_t next64(void) {
  uint64_t z = (mix_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* BF16 bit patterns: "weights" have a random sign and mantissa and an
 * exponent within a few steps of 2^-6, with a share `rare` (per 1024) of
 * exponents anywhere; "uniform" draws all 16 bits; "const" repeats 1.0. */
enum { W_WEIGHTS, W_UNIFORM, W_CONST };
static void fill(uint16_t *w, uint64_t n, int kind, unsigned rare) {
  for (uint64_t i = 0; i < n; ++i) {
    const uint64_t r = next64();
    if (kind == W_UNIFORM) {
      w[i] = (uint16_t)r;
    } else if (kind == W_CONST) {
      w[i] = 0x3F80;
    } else {
      const uint32_t sign = (uint32_t)(r >> 63) << 15;
      uint32_t ex = 121u + (uint32_t)((r >> 8) % 6u);
      if ((r >> 20) % 1024u < rare) ex = (uint32_t)((r >> 32) & 0xFFu);
      w[i] = (uint16_t)(sign | ex << 7 | (uint32_t)(r & 0x7Fu));
    }
  }
}

static uint8_t *encode(int layout, int flags, const uint16_t *w, uint64_t n, uint64_t *size) {
  /* room for the largest container: header, 4 bytes of streams per weight
   * (codes, raw, a 4-byte position and a 2-byte symbol if every weight
   * escapes, over-counted), the index and padding */
  const uint64_t cap = 1024u + 16u * n;
  uint8_t *c = (uint8_t *)malloc(cap);
  const int rc = orc_encode_flags(layout, flags, w, n, c, cap, size);
  CHECK(rc == ORC_OK, "encode layout %d flags %d n %llu: %d", layout, flags, (unsigned long long)n, rc);
  return c;
}

static void round_trip(int layout, int flags, int kind, unsigned rare, uint64_t n) {
  uint16_t *w = (uint16_t *)malloc((n ? n : 1) * 2);
  fill(w, n, kind, rare);
  uint64_t size = 0;
  uint8_t *c = encode(layout, flags, w, n, &size);
  uint64_t total = 0;
  int nd;
  uint64_t nn, ne, off[6];
  uint16_t dict[16];
  CHECK(orc_header_info(c, size, &layout, &nd, &nn, &ne, dict, off) == ORC_OK, "header_info");
  CHECK(orc_container_size_flags(layout, flags, n, ne, &total) == ORC_OK && total == size,
        "size formula %llu vs %llu", (unsigned long long)total, (unsigned long long)size);
  uint16_t *d = (uint16_t *)malloc((n ? n : 1) * 2);
  CHECK(orc_decode(c, size, d, n) == ORC_OK, "decode");
  CHECK(n == 0 || memcmp(d, w, n * 2) == 0, "round trip layout %d flags %d n %llu", layout, flags,
        (unsigned long long)n);
  if (n) {
    double bpw, pbpw;
    CHECK(orc_bits_per_weight(c, size, &bpw, &pbpw) == ORC_OK && pbpw <= bpw, "bits per weight");
  }
  /* a buffer one short of the container (an allocation of that size, so a
   * read past it is a sanitizer report), and one weight too small for out */
  if (size > 0) {
    uint8_t *shortc = (uint8_t *)malloc(size - 1);
    memcpy(shortc, c, size - 1);
    CHECK(orc_decode(shortc, size - 1, d, n) == ORC_E_CORRUPT, "short buffer accepted");
    free(shortc);
  }
  if (n) CHECK(orc_decode(c, size, d, n - 1) == ORC_E_ARG, "small output accepted");
  free(d);
  free(c);
  free(w);
}

/* Every byte of a small container with one bit flipped (bit k % 8 of byte
 * k): decode answers OK or CORRUPT.  A container carries no checksum of its
 * own, so a flip can leave a valid container: a changed dictionary symbol,
 * or a weight count that keeps every stream's padded length (then up to 16
 * more weights decode, hence the room in `d`). */
static void flips(int layout, int flags, int kind, unsigned rare, uint64_t n, uint64_t *seen_ok,
                  uint64_t *seen_corrupt) {
  uint16_t *w = (uint16_t *)malloc((n ? n : 1) * 2);
  fill(w, n, kind, rare);
  uint64_t size = 0;
  uint8_t *c = encode(layout, flags, w, n, &size);
  uint8_t *bad = (uint8_t *)malloc(size);
  uint16_t *d = (uint16_t *)malloc((n + 64) * 2);
  for (uint64_t k = 0; k < size; ++k) {
    memcpy(bad, c, size);
    bad[k] ^= (uint8_t)(1u << (k % 8));
    const int rc = orc_decode(bad, size, d, n + 64);
    CHECK(rc == ORC_OK || rc == ORC_E_CORRUPT, "flip at %llu: %d", (unsigned long long)k, rc);
    if (rc == ORC_OK) ++*seen_ok;
    else ++*seen_corrupt;
  }
  free(d);
  free(bad);
  free(c);
  free(w);
}

int main(void) {
  mix_state = 20240611ull;
  static const uint64_t sizes[] = {0, 1, 15, 2047, 2048, 2049, 8191, 8192, 3 * 8192 + 5, 70001};
  int n_rt = 0;
  for (int layout = 0; layout <= 2; ++layout)
    for (int flags = 0; flags <= (layout == ORC_LAYOUT_RAW ? 0 : ORC_FLAG_COMPACT); ++flags)
      for (int kind = 0; kind < 3; ++kind)
        for (size_t s = 0; s < sizeof sizes / sizeof sizes[0]; ++s) {
          round_trip(layout, flags, kind, 8, sizes[s]);
          ++n_rt;
        }
  printf("round trips: %d\n", n_rt);

  uint64_t ok = 0, corrupt = 0;
  for (int layout = 0; layout <= 2; ++layout)
    for (int flags = 0; flags <= (layout == ORC_LAYOUT_RAW ? 0 : ORC_FLAG_COMPACT); ++flags) {
      flips(layout, flags, W_WEIGHTS, 40, 3000, &ok, &corrupt);
      flips(layout, flags, W_UNIFORM, 0, 700, &ok, &corrupt);
    }
  printf("flipped containers: %llu decoded, %llu corrupt\n", (unsigned long long)ok,
         (unsigned long long)corrupt);

  /* headers of random bytes behind a valid magic and version */
  int rejected = 0;
  for (int t = 0; t < 20000; ++t) {
    uint8_t c[4096];
    for (int k = 0; k < (int)sizeof c; ++k) c[k] = (uint8_t)next64();
    memcpy(c, "WC16", 4); /* the container's magic, then version 2 */
    c[4] = 2;
    c[5] = 0;
    c[6] = (uint8_t)(t % 3); /* a valid layout */
    uint16_t d[64];
    const int rc = orc_decode(c, sizeof c, d, 64);
    CHECK(rc == ORC_E_CORRUPT || rc == ORC_E_ARG || rc == ORC_OK, "random bytes: %d", rc);
    rejected += rc != ORC_OK;
  }
  printf("random headers rejected: %d of 20000\n", rejected);

  /* histogram, dictionary, layout choice and GEMV on ragged shapes */
  static const uint64_t shapes[][2] = {{0, 0}, {0, 5}, {3, 0}, {1, 1}, {7, 33}, {64, 2049}, {5, 4097}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
    const uint64_t rows = shapes[s][0], cols = shapes[s][1], n = rows * cols;
    for (uint32_t batch = 1; batch <= 4; batch += 3) {
      uint16_t *W = (uint16_t *)malloc((n ? n : 1) * 2);
      uint16_t *x = (uint16_t *)malloc((batch * cols > 0 ? batch * cols : 1) * 2);
      fill(W, n, W_WEIGHTS, 0); /* finite values: products stay in fp32's range */
      fill(x, batch * cols, W_WEIGHTS, 0);
      float *y = (float *)malloc((batch * rows > 0 ? batch * rows : 1) * sizeof(float));
      double *y64 = (double *)malloc((batch * rows > 0 ? batch * rows : 1) * sizeof(double));
      double *a64 = (double *)malloc((batch * rows > 0 ? batch * rows : 1) * sizeof(double));
      CHECK(orc_gemv_f32(W, rows, cols, x, batch, y) == ORC_OK, "gemv f32");
      CHECK(orc_gemv_f64(W, rows, cols, x, batch, y64, a64) == ORC_OK, "gemv f64");
      /* BF16 x BF16 products are exact in fp32, so only the cols - 1
       * additions round: |f32 - exact| <= (cols - 1) u / (1 - (cols - 1) u)
       * sum |W x| with u = 2^-24, and the fp64 sum is within 2^-40 of exact */
      const double u = 1.0 / 16777216.0, m = cols ? (double)(cols - 1) : 0.0;
      for (uint64_t i = 0; i < batch * rows; ++i) {
        const double err = (double)y[i] - y64[i];
        CHECK((err < 0 ? -err : err) <= (m * u / (1 - m * u) + 1e-12) * a64[i], "gemv f32 vs f64 at %llu",
              (unsigned long long)i);
      }
      for (int layout = 0; layout <= 1; ++layout) {
        uint64_t counts[512];
        uint16_t dict[16];
        int nd;
        uint64_t ne;
        CHECK(orc_histogram(layout, W, n, counts) == ORC_OK, "histogram");
        CHECK(orc_dictionary(layout, counts, n, dict, &nd, &ne) == ORC_OK && ne <= n, "dictionary");
      }
      int lay;
      CHECK(orc_choose_layout(W, n, &lay) == ORC_OK && lay >= 0 && lay <= 2, "choose layout");
      free(a64);
      free(y64);
      free(y);
      free(x);
      free(W);
    }
  }
  printf("gemv shapes: %d\n", (int)(sizeof shapes / sizeof shapes[0]));
  printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
