/*
 * wc.h — C ABI of libwc: lossless BF16 sign+exponent coding, exact decode,
 * and decode fused into GEMV, on AMD Instinct MI355X (gfx950).
 *
 * What the operations are (page title, section):
 *  [P2] "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está listo
 *       para producción?" — "¿Qué significa “sin pérdida” para los pesos de
 *       un LLM?" (lossless = every source bit rebuilt; exact BF16 may be
 *       rebuilt in registers or shared memory and used at once in the matrix
 *       product) and "¿Qué demostró realmente el experimento con GLM-5.2?"
 *       (BF16 = sign 1 + exponent 8 + mantissa 7; short codes for frequent
 *       sign+exponent symbols; rare ones in an exact escape stream).
 *  [P3] "Prueba de GLM-5.2 reduce la memoria BF16 en casi un 25%" —
 *       "Cómo funciona la compresión" (K15: 9-bit symbol -> 4-bit code into a
 *       15-entry table, exact escapes, 7-bit mantissa raw, bits/weight with
 *       all overhead; byte-split: high byte from dictionary + code indices +
 *       escape stream, low byte unchanged) and "Qué queda por demostrar"
 *       (a dense 12-bit prototype rebuilt codes in registers and was timed
 *       against a BF16 GEMV, with the escape correction kept apart).
 *
 * Container (all integers little-endian; every stream starts at a 16-byte
 * aligned offset; gaps and tails are zero):
 *   [0,128)          wc_header below
 * Byte-split and K15 (layouts 0 and 1):
 *   off_codes (128)  4-bit codes, ceil(n/2) bytes; weight i in byte i/2, the
 *                    low nibble when i is even; code k < n_dict selects
 *                    dict[k]; code 15 marks an escape
 *   off_raw          byte-split: the low byte of every weight, n bytes;
 *                    K15: the 7-bit mantissas as one LSB-first bitstream,
 *                    mantissa i at stream bits [7i, 7i+7), ceil(7n/8) bytes
 *   off_esc_pos      n_esc u32 positions (flat weight index), ascending;
 *                    empty in the compact form (flags & WC_FLAG_COMPACT),
 *                    where the k-th code-15 weight is the k-th record
 *   off_esc_sym      n_esc symbols: u8 (byte-split) or u16 (K15)
 *   off_esc_idx      escape index, only when n_esc > 0: for j = 0..T with
 *                    T = ceil(n / WC_INDEX_TILE), u32 entry j = the number of
 *                    escapes at positions below j * WC_INDEX_TILE (entry T =
 *                    n_esc), so a kernel finds the first escape record of any
 *                    tile with one load instead of a search of the positions
 *   total_bytes      end of the container
 * Raw (layout 2, a per-tensor fallback for tensors that do not code below
 * 16 bits/weight): n_dict = n_esc = 0, dictionary zero, an empty code
 * stream, and the raw stream at off_raw = 128 holds the n BF16 bit patterns
 * as u16; the escape streams are empty (all later offsets = total_bytes).
 * Symbols: byte-split s = b >> 8 (sign + exponent[7:1]); K15 s = b >> 7
 * (sign + exponent).  A weight is rebuilt as (s << 8) | low byte, or
 * (s << 7) | mantissa.  The dictionary holds the min(15, #distinct) most
 * frequent symbols of the tensor, ties to the smaller symbol; its order is
 * the code order.  Weights are the tensor's row-major flat order; a matrix
 * W[rows][cols] multiplies as y = W x (x has cols entries).
 *
 * Conventions for every call:
 *  - Device pointers (d_*) are caller-owned device memory; the library
 *    allocates nothing and keeps no pointer after returning.  Host pointers
 *    (h, h_out, results) are caller-owned host memory.
 *  - d_w, d_container, d_out, d_x must be 16-byte aligned; d_y 4-byte.
 *  - `stream` is a hipStream_t (NULL = the null stream).  All device work is
 *    enqueued on it in order and returns without waiting, except
 *    wc_build_dict, which waits for `stream` once (it reads back 48 bytes, or
 *    96 under WC_LAYOUT_AUTO).
 *  - Return value: WC_OK or a negative WC_E_* code; nothing is enqueued when
 *    an argument check fails.  A device fault shows up at the caller's next
 *    synchronisation.  No call aborts or throws.
 */
#ifndef WC_H
#define WC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WC_LAYOUT_BYTESPLIT 0
#define WC_LAYOUT_K15 1
#define WC_LAYOUT_RAW 2  /* fallback: the BF16 bit patterns as they are */
#define WC_LAYOUT_AUTO 3 /* wc_build_dict only: the smallest of the three */

#define WC_OK 0
#define WC_E_ARG (-1)         /* null pointer, misalignment, bad size/shape */
#define WC_E_SIZE (-2)        /* n >= 2^32, or a buffer smaller than needed */
#define WC_E_CORRUPT (-3)     /* header fails validation */
#define WC_E_HIP (-4)         /* a HIP call or kernel launch failed */
#define WC_E_UNSUPPORTED (-5) /* batch outside 1..WC_MAX_BATCH */
#define WC_E_IO (-6)          /* a file could not be opened, read or written */

#define WC_MAGIC 0x36314357u /* bytes "WC16" */
#define WC_VERSION 2u
#define WC_HEADER_BYTES 128u
#define WC_INDEX_TILE 2048u /* weights per escape-index entry */
#define WC_MAX_BATCH 256u

/* Header flags.  WC_FLAG_COMPACT: the escape stream holds the symbols only,
 * in weight order, and the k-th weight whose code is 15 takes the k-th
 * symbol (no position stream: off_esc_sym == off_esc_pos).  Coded layouts
 * only.  Request it by OR-ing WC_COMPACT into wc_build_dict's layout. */
#define WC_FLAG_COMPACT 1u
#define WC_COMPACT 0x10

/* Scratch bytes wc_build_dict and wc_encode need for n weights: 20528, plus
 * 16 per 8192-weight block for its escape count, first record and tile
 * counts, plus 6 * WC_STAGE_SYMBOLS per block, where encode stages the
 * escape records (2-byte symbol, 4-byte position) of blocks that have at
 * most WC_STAGE_SYMBOLS of them (0.19 bytes/weight). */
#define WC_STAGE_SYMBOLS 256u
#define WC_WORKSPACE_BYTES(n) \
  ((size_t)20528 + (size_t)(16u + 6u * WC_STAGE_SYMBOLS) * (((uint64_t)(n) + 8191u) / 8192u))

/* The first 128 bytes of every container, byte for byte. */
typedef struct wc_header {
  uint32_t magic;       /* WC_MAGIC */
  uint16_t version;     /* WC_VERSION */
  uint8_t layout;       /* WC_LAYOUT_* */
  uint8_t n_dict;       /* dictionary entries, 0..15 */
  uint64_t n;           /* weights, < 2^32 */
  uint64_t n_esc;       /* escape records */
  uint16_t dict[16];    /* symbols by code; entries n_dict..15 are 0 */
  uint64_t off_codes;   /* = 128 */
  uint64_t off_raw;     /* = pad16(128 + ceil(n/2)) */
  uint64_t off_esc_pos; /* = pad16(off_raw + raw bytes) */
  uint64_t off_esc_sym; /* = pad16(off_esc_pos + 4 n_esc) */
  uint64_t total_bytes; /* = pad16(off_esc_idx + 4 (T + 1)), or off_esc_idx when n_esc == 0 */
  uint64_t off_esc_idx; /* = pad16(off_esc_sym + symbol bytes) */
  uint8_t flags;        /* WC_FLAG_* */
  uint8_t reserved[23]; /* zero */
} wc_header;

/*
 * Per-tensor dictionary [P3 "Cómo funciona la compresión"; P2 "¿Qué
 * demostró…"]: counts the sign+exponent symbols of d_w[0..n) (BF16 bit
 * patterns), takes the top 15 as the dictionary, and fills *h_out with the
 * complete header of the container wc_encode will write (escape count,
 * stream offsets and total size included), so the caller can allocate it.
 * layout WC_LAYOUT_AUTO counts both symbol kinds in the same pass and
 * returns the header of whichever of byte-split, K15 and raw gives the
 * smallest container (ties to the lower layout number); WC_LAYOUT_RAW needs
 * no device work and does not wait.  The pages ask for a BF16 fallback
 * where the coding does not pay (page "Compresión de pesos LLM sin pérdida
 * vs 8-bit GGUF…", section "Preguntas para un vendor o equipo de
 * investigación").  layout | WC_COMPACT gives a coded layout the compact
 * escape form (WC_FLAG_COMPACT; the raw layout ignores it).
 * d_work: WC_WORKSPACE_BYTES(n) bytes of device scratch (contents ignored
 * and overwritten).  Waits for `stream`.  n == 0 is allowed (empty tensor).
 */
int wc_build_dict(int layout, const uint16_t *d_w, uint64_t n, void *d_work,
                  size_t work_bytes, void *stream, wc_header *h_out);

/*
 * Encode [P3 "Cómo funciona la compresión"]: writes the whole container for
 * d_w[0..h->n) — header, codes, raw stream, escape positions and symbols —
 * into d_container[0..h->total_bytes) (with the escape index when there are
 * escapes).  *h must be the header wc_build_dict
 * returned for the same weights (checked for consistency; a header whose
 * escape count does not match the data yields a container that fails to
 * decode).  container_bytes >= h->total_bytes; d_work as for wc_build_dict.
 */
int wc_encode(const wc_header *h, const uint16_t *d_w, uint8_t *d_container,
              size_t container_bytes, void *d_work, size_t work_bytes,
              void *stream);

/*
 * wc_encode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same container as wc_encode for the same header and
 * weights.  Its scratch (each 8192-weight block's escape count and first
 * record) is a fixed device array of the library, 8 * 2^18 + 32 bytes
 * (2 MiB) on each GPU it runs on, held until the process ends; every call
 * writes what it reads there first.  It stages no escape symbols, so the
 * weights of blocks with escapes are read twice (wc_encode reads them once
 * when a block has at most WC_STAGE_SYMBOLS escapes).  h->n >
 * WC_NOALLOC_MAX_N -> WC_E_SIZE.
 * All calls on one GPU share that array: calls that overlap on one GPU
 * (other streams, other host threads) race and must not be issued; calls in
 * one stream's order are safe.  Allocates nothing (no hipMalloc, hipFree or
 * allocating library call); the first call on a device looks up the
 * array's device address.
 */
#define WC_NOALLOC_MAX_N (1ull << 31)
int wc_encode_noalloc(const wc_header *h, const uint16_t *d_w, uint8_t *d_container,
                      size_t container_bytes, void *stream);

/*
 * Exact decode [P3 "Cómo funciona la compresión"; P2 "¿Qué significa “sin
 * pérdida”…"]: rebuilds the n BF16 bit patterns into d_out[0..n).  *h is the
 * host copy of the container's header (validated: WC_E_CORRUPT).  Escape
 * index entries are clamped to [0, n_esc], and escape records whose position
 * lies outside the tile being decoded, or past n_esc, are ignored, so a
 * corrupt stream body cannot make the kernel read or write outside the
 * container and d_out.  In the compact form (WC_FLAG_COMPACT) the k-th
 * code-15 weight takes the k-th symbol, placed by its rank in the tile.
 */
int wc_decode(const wc_header *h, const uint8_t *d_container,
              size_t container_bytes, uint16_t *d_out, void *stream);

/*
 * Decode fused into GEMV [P2 "¿Qué significa “sin pérdida”…"; P3 "Qué queda
 * por demostrar"]: y[b][r] = sum_c W[r][c] * x[b][c] with W the container's
 * weights viewed as [rows][cols] (rows * cols == h->n), rebuilt in registers
 * with escapes applied and never written to memory.  d_x: BF16 [batch][cols];
 * d_y: fp32 [batch][rows].  Products are exact (BF16 x BF16), sums are fp32
 * in an order that differs from a sequential loop.  batch in
 * 1..WC_MAX_BATCH, else WC_E_UNSUPPORTED.  In the prefill regime, where
 * the pages' closest prior art is a fused decompression-GEMM [P2 "¿Cómo
 * encaja con los sistemas anteriores?"], each rebuilt weight is used by up
 * to 128 input rows on the matrix cores: above 32 input rows (above 16 on
 * tensors of 2^26 weights or more) when cols is a multiple of 128.  Other
 * batches above 16 run 16 input rows at a time.  Both escape forms are
 * taken; in the compact one (WC_FLAG_COMPACT) a row that starts inside an
 * index tile finds its first record by counting the code-15 marks from the
 * tile start.
 */
int wc_decode_gemv(const wc_header *h, const uint8_t *d_container,
                   size_t container_bytes, uint64_t rows, uint64_t cols,
                   const uint16_t *d_x, uint32_t batch, float *d_y,
                   void *stream);

/*
 * Plain BF16 GEMV, the comparison the pages time the fused kernel against
 * [P3 "Qué queda por demostrar"]: same shapes, types and reduction tree as
 * wc_decode_gemv, with W read as uncompressed BF16 [rows][cols].
 */
int wc_gemv_bf16(const uint16_t *d_w, uint64_t rows, uint64_t cols,
                 const uint16_t *d_x, uint32_t batch, float *d_y, void *stream);

/*
 * Accounting [P3 "Cómo funciona la compresión": bits per weight with all
 * overhead included]: *bpw = 8 * total_bytes / n (header, dictionary,
 * streams, padding); *payload_bpw = 8 * (codes + raw + escape bytes) / n,
 * the escape bytes being positions, symbols and the escape index.
 * Host only.  n == 0 -> WC_E_ARG.
 */
int wc_bits_per_weight(const wc_header *h, double *bpw, double *payload_bpw);

/*
 * ---- Serialized artifact (host only) --------------------------------------
 * The pages ask that a saving be shown on a serialized artifact that holds
 * the metadata and the escapes, that every tensor be decoded from what was
 * delivered and compared, and that corruption have a defined outcome (page
 * "Compresión de pesos LLM sin pérdida vs 8-bit GGUF…", sections "¿Está
 * listo para producción el resultado de GLM-5.2?" and "Preguntas para un
 * vendor o equipo de investigación").
 *
 * File (little-endian): a 64-byte file header, a table of 256-byte entries,
 * then the containers, each at a 4096-byte aligned offset, gaps zero.
 *   file header: magic "WCA1", version u16 = 1, u16 0, count u32, u32 0,
 *     table offset u64 (64), data offset u64, file bytes u64, 20 zero bytes,
 *     CRC-32 of bytes [0, 60) at 60.
 *   entry: name (96 bytes, NUL-terminated, NUL-padded), ndim u32 (1..4),
 *     layout u32, shape u64[4] (unused dims 0, product = n), container offset
 *     u64 and bytes u64, the source's CRC-32 (of its n BF16 values as
 *     little-endian u16, given by the writer), the six stream CRC-32s
 *     (wc_container_crcs), zeros, and at 252 the CRC-32 of bytes [0, 252).
 * Reading checks every CRC, the container header and that the entry agrees
 * with it: any mismatch is WC_E_CORRUPT, a short or unreadable file WC_E_IO
 * or WC_E_CORRUPT.  The decoded tensor is then compared with src_crc by the
 * caller (it is the only check of the rebuilt weights themselves).
 */
#define WC_ARTIFACT_MAGIC 0x31414357u /* bytes "WCA1" */
#define WC_ARTIFACT_ALIGN 4096u
#define WC_ARTIFACT_NAME 96u

typedef struct wc_artifact_info {
  char name[WC_ARTIFACT_NAME];
  uint32_t ndim, layout;
  uint64_t shape[4];
  uint64_t offset, bytes; /* the container inside the file */
  uint32_t src_crc;       /* CRC-32 of the source BF16 values */
  uint32_t stream_crc[6]; /* header, codes, raw, escape positions, symbols, index */
  uint32_t reserved;
} wc_artifact_info;

/* CRC-32 (IEEE 802.3, reflected, polynomial 0xEDB88320), continued from
 * `crc` (0 to start) over data[0, len); the same value zlib's crc32 gives. */
uint32_t wc_crc32(uint32_t crc, const void *data, size_t len);

/* CRC-32 of each of a container's six regions, which cover every byte once:
 * [0,128) header, [off_codes, off_raw), [off_raw, off_esc_pos),
 * [off_esc_pos, off_esc_sym), [off_esc_sym, off_esc_idx),
 * [off_esc_idx, total_bytes).  h_container is host memory of `bytes` bytes;
 * its header is validated (WC_E_CORRUPT), bytes >= total_bytes (WC_E_SIZE). */
int wc_container_crcs(const uint8_t *h_container, size_t bytes, uint32_t crc[6]);

/* Writes `count` containers (host memory, each validated) with their names,
 * shapes and source CRCs into a new file at `path` (replaced if present). */
int wc_artifact_write(const char *path, uint32_t count, const char *const *names,
                      const uint32_t *ndims, const uint64_t *shapes /* [count][4] */,
                      const uint8_t *const *h_containers, const uint64_t *container_bytes,
                      const uint32_t *src_crcs);

/* Number of entries, after checking the file header, every entry's CRC, that
 * each container sits where the writer places it (the data offset, then the
 * next 4096-byte boundary after the previous one; the file ends with the last)
 * and that every gap byte is zero: with the CRCs, any changed byte of the file
 * is reported as WC_E_CORRUPT. */
int wc_artifact_count(const char *path, uint32_t *count);

/* Entry i's metadata (file header and entry checked). */
int wc_artifact_entry(const char *path, uint32_t i, wc_artifact_info *out);

/* Reads container i into h_buf (at least info.bytes bytes) and checks its
 * header against the entry and every stream CRC. */
int wc_artifact_read(const char *path, uint32_t i, uint8_t *h_buf, size_t buf_bytes);

#ifdef __cplusplus
}
#endif
#endif /* WC_H */
