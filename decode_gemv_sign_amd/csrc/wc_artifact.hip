// wc_artifact.hip — host-only: CRC-32, per-stream container checksums and the
// serialized multi-tensor artifact (file layout in include/wc.h).
//
// The pages ask that a saving be shown on a serialized artifact with its
// metadata and escapes, that every tensor be decoded from what was delivered
// and compared with its source, and that corruption have a defined outcome
// (page "Compresión de pesos LLM sin pérdida vs 8-bit GGUF: ¿qué está listo
// para producción?", sections "¿Está listo para producción el resultado de
// GLM-5.2?" and "Preguntas para un vendor o equipo de investigación").  Here
// every byte of the file is either under a CRC-32 (the file header, each
// table entry and each of a container's six regions) or a gap byte that must
// be zero where the writer puts it; a reader reports any mismatch as
// WC_E_CORRUPT before a container reaches the GPU.
#include <stdio.h>
#include <string.h>
#include <sys/stat.h>

#include <string>
#include <vector>

#include "wc_common.h"

namespace {

// ---- CRC-32 (IEEE 802.3): reflected, polynomial 0xEDB88320 ---------------
// Slice-by-8: table k maps a byte to the CRC of that byte followed by k zero
// bytes, so eight bytes are folded per step.
struct CrcTables {
  uint32_t t[8][256];
  CrcTables() {
    for (uint32_t i = 0; i < 256; ++i) {
      uint32_t c = i;
      for (int k = 0; k < 8; ++k) c = (c & 1u) ? 0xEDB88320u ^ (c >> 1) : c >> 1;
      t[0][i] = c;
    }
    for (int k = 1; k < 8; ++k)
      for (uint32_t i = 0; i < 256; ++i) t[k][i] = (t[k - 1][i] >> 8) ^ t[0][t[k - 1][i] & 0xFFu];
  }
};

const CrcTables& crc_tables() {
  static const CrcTables tables;  // built once, thread-safe
  return tables;
}

uint32_t crc32_update(uint32_t crc, const uint8_t* p, size_t len) {
  const CrcTables& T = crc_tables();
  uint32_t c = ~crc;
  while (len >= 8) {
    const uint32_t lo = c ^ ((uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24);
    const uint32_t hi = (uint32_t)p[4] | (uint32_t)p[5] << 8 | (uint32_t)p[6] << 16 | (uint32_t)p[7] << 24;
    c = T.t[7][lo & 0xFFu] ^ T.t[6][(lo >> 8) & 0xFFu] ^ T.t[5][(lo >> 16) & 0xFFu] ^ T.t[4][lo >> 24] ^
        T.t[3][hi & 0xFFu] ^ T.t[2][(hi >> 8) & 0xFFu] ^ T.t[1][(hi >> 16) & 0xFFu] ^ T.t[0][hi >> 24];
    p += 8;
    len -= 8;
  }
  while (len--) c = T.t[0][(c ^ *p++) & 0xFFu] ^ (c >> 8);
  return ~c;
}

// ---- little-endian fields -------------------------------------------------

void put(uint8_t* p, uint64_t v, int bytes) {
  for (int k = 0; k < bytes; ++k) p[k] = (uint8_t)(v >> (8 * k));
}
uint64_t get(const uint8_t* p, int bytes) {
  uint64_t v = 0;
  for (int k = 0; k < bytes; ++k) v |= (uint64_t)p[k] << (8 * k);
  return v;
}

constexpr uint32_t kFileHeader = 64, kEntry = 256, kVersion = 1;

uint64_t align_up(uint64_t x) { return (x + WC_ARTIFACT_ALIGN - 1) / WC_ARTIFACT_ALIGN * WC_ARTIFACT_ALIGN; }

// The six regions of a container (wc_container_crcs).
void regions(const wc_header& h, uint64_t lo[6], uint64_t hi[6]) {
  const uint64_t b[7] = {0, WC_HEADER_BYTES, h.off_raw, h.off_esc_pos, h.off_esc_sym, h.off_esc_idx,
                         h.total_bytes};
  for (int k = 0; k < 6; ++k) {
    lo[k] = b[k];
    hi[k] = b[k + 1];
  }
}

int crcs_of(const uint8_t* c, size_t bytes, wc_header* h_out, uint32_t crc[6]) {
  if (bytes < WC_HEADER_BYTES) return WC_E_CORRUPT;
  wc_header h;
  memcpy(&h, c, sizeof h);
  const int v = wc::validate_header(&h);
  if (v != WC_OK) return v;
  if (bytes < h.total_bytes) return WC_E_SIZE;
  uint64_t lo[6], hi[6];
  regions(h, lo, hi);
  for (int k = 0; k < 6; ++k) crc[k] = crc32_update(0, c + lo[k], (size_t)(hi[k] - lo[k]));
  if (h_out) *h_out = h;
  return WC_OK;
}

// An open file, closed on scope exit.
struct File {
  FILE* f = nullptr;
  File(const char* path, const char* mode) : f(fopen(path, mode)) {}
  ~File() {
    if (f) fclose(f);
  }
  bool read_at(uint64_t off, void* dst, size_t n) {
    return fseeko(f, (off_t)off, SEEK_SET) == 0 && fread(dst, 1, n, f) == n;
  }
};

// File header checks: magic, version, CRC, the table and data placement,
// and the recorded size against the file's own.
int read_file_header(File& file, uint32_t* count, uint64_t* data_off, uint64_t* file_bytes) {
  uint8_t fh[kFileHeader];
  if (!file.f) return WC_E_IO;
  if (fseeko(file.f, 0, SEEK_END) != 0) return WC_E_IO;
  const off_t size = ftello(file.f);
  if (size < (off_t)kFileHeader) return WC_E_CORRUPT;
  if (!file.read_at(0, fh, kFileHeader)) return WC_E_IO;
  if (get(fh + 60, 4) != crc32_update(0, fh, 60)) return WC_E_CORRUPT;
  if (get(fh, 4) != WC_ARTIFACT_MAGIC || get(fh + 4, 2) != kVersion || get(fh + 6, 2) != 0 ||
      get(fh + 12, 4) != 0)
    return WC_E_CORRUPT;
  for (int k = 40; k < 60; ++k)
    if (fh[k]) return WC_E_CORRUPT;
  const uint64_t n = get(fh + 8, 4);
  if (get(fh + 16, 8) != kFileHeader) return WC_E_CORRUPT;
  const uint64_t doff = get(fh + 24, 8);
  if (doff != align_up(kFileHeader + kEntry * n)) return WC_E_CORRUPT;
  if (get(fh + 32, 8) != (uint64_t)size) return WC_E_CORRUPT;
  if (n && (uint64_t)size < doff) return WC_E_CORRUPT;
  *count = (uint32_t)n;
  *data_off = doff;
  *file_bytes = (uint64_t)size;
  return WC_OK;
}

int read_entry(File& file, uint32_t i, wc_artifact_info* out) {
  uint32_t count;
  uint64_t doff, fsize;
  int st = read_file_header(file, &count, &doff, &fsize);
  if (st != WC_OK) return st;
  if (i >= count) return WC_E_ARG;
  uint8_t e[kEntry];
  if (!file.read_at(kFileHeader + (uint64_t)kEntry * i, e, kEntry)) return WC_E_CORRUPT;
  if (get(e + 252, 4) != crc32_update(0, e, 252)) return WC_E_CORRUPT;
  wc_artifact_info info;
  memset(&info, 0, sizeof info);
  memcpy(info.name, e, WC_ARTIFACT_NAME);
  if (memchr(info.name, 0, WC_ARTIFACT_NAME) == nullptr) return WC_E_CORRUPT;
  info.ndim = (uint32_t)get(e + 96, 4);
  info.layout = (uint32_t)get(e + 100, 4);
  for (int k = 0; k < 4; ++k) info.shape[k] = get(e + 104 + 8 * k, 8);
  info.offset = get(e + 136, 8);
  info.bytes = get(e + 144, 8);
  info.src_crc = (uint32_t)get(e + 152, 4);
  for (int k = 0; k < 6; ++k) info.stream_crc[k] = (uint32_t)get(e + 156 + 4 * k, 4);
  for (int k = 180; k < 252; ++k)
    if (e[k]) return WC_E_CORRUPT;
  if (info.ndim < 1 || info.ndim > 4 || info.layout > WC_LAYOUT_RAW) return WC_E_CORRUPT;
  for (uint32_t k = info.ndim; k < 4; ++k)
    if (info.shape[k]) return WC_E_CORRUPT;
  if (info.offset % WC_ARTIFACT_ALIGN || info.offset < doff || info.bytes < WC_HEADER_BYTES)
    return WC_E_CORRUPT;
  if (info.offset > fsize || info.bytes > fsize - info.offset) return WC_E_CORRUPT;
  *out = info;
  return WC_OK;
}

}  // namespace

extern "C" uint32_t wc_crc32(uint32_t crc, const void* data, size_t len) {
  if (!data || !len) return crc;
  return crc32_update(crc, (const uint8_t*)data, len);
}

extern "C" int wc_container_crcs(const uint8_t* h_container, size_t bytes, uint32_t crc[6]) {
  if (!h_container || !crc) return WC_E_ARG;
  return crcs_of(h_container, bytes, nullptr, crc);
}

extern "C" int wc_artifact_write(const char* path, uint32_t count, const char* const* names,
                                 const uint32_t* ndims, const uint64_t* shapes,
                                 const uint8_t* const* h_containers,
                                 const uint64_t* container_bytes, const uint32_t* src_crcs) {
  if (!path || (count && (!names || !ndims || !shapes || !h_containers || !container_bytes || !src_crcs)))
    return WC_E_ARG;
  if ((uint64_t)count * kEntry > (1ull << 40)) return WC_E_SIZE;
  std::vector<uint8_t> table((size_t)count * kEntry, 0);
  std::vector<uint64_t> offs(count), sizes(count);
  uint64_t at = align_up(kFileHeader + (uint64_t)kEntry * count);
  const uint64_t data_off = at;
  for (uint32_t i = 0; i < count; ++i) {
    if (!names[i] || !h_containers[i]) return WC_E_ARG;
    const size_t len = strlen(names[i]);
    if (len >= WC_ARTIFACT_NAME) return WC_E_ARG;
    if (ndims[i] < 1 || ndims[i] > 4) return WC_E_ARG;
    wc_header h;
    uint32_t crc[6];
    const int st = crcs_of(h_containers[i], (size_t)container_bytes[i], &h, crc);
    if (st != WC_OK) return st;
    uint64_t prod = 1;
    for (uint32_t k = 0; k < 4; ++k) {
      const uint64_t d = shapes[4 * (size_t)i + k];
      if (k >= ndims[i] && d != 0) return WC_E_ARG;  // unused dimensions are 0
      if (k < ndims[i]) prod *= d;
    }
    if (prod != h.n) return WC_E_ARG;
    uint8_t* e = table.data() + (size_t)kEntry * i;
    memcpy(e, names[i], len);
    put(e + 96, ndims[i], 4);
    put(e + 100, h.layout, 4);
    for (int k = 0; k < 4; ++k) put(e + 104 + 8 * k, shapes[4 * (size_t)i + k], 8);
    offs[i] = at;
    sizes[i] = h.total_bytes;
    put(e + 136, at, 8);
    put(e + 144, h.total_bytes, 8);
    put(e + 152, src_crcs[i], 4);
    for (int k = 0; k < 6; ++k) put(e + 156 + 4 * k, crc[k], 4);
    put(e + 252, crc32_update(0, e, 252), 4);
    at = align_up(at + h.total_bytes);
  }
  const uint64_t file_bytes = count ? offs[count - 1] + sizes[count - 1] : kFileHeader;
  uint8_t fh[kFileHeader];
  memset(fh, 0, sizeof fh);
  put(fh, WC_ARTIFACT_MAGIC, 4);
  put(fh + 4, kVersion, 2);
  put(fh + 8, count, 4);
  put(fh + 16, kFileHeader, 8);
  put(fh + 24, data_off, 8);
  put(fh + 32, file_bytes, 8);
  put(fh + 60, crc32_update(0, fh, 60), 4);

  // written to a temporary name, then renamed over `path`
  const std::string tmp = std::string(path) + ".tmp";
  {
    File file(tmp.c_str(), "wb");
    if (!file.f) return WC_E_IO;
    bool ok = fwrite(fh, 1, kFileHeader, file.f) == kFileHeader;
    ok = ok && (table.empty() || fwrite(table.data(), 1, table.size(), file.f) == table.size());
    static const uint8_t zeros[WC_ARTIFACT_ALIGN] = {0};
    uint64_t pos = kFileHeader + (uint64_t)table.size();
    for (uint32_t i = 0; ok && i < count; ++i) {
      while (ok && pos < offs[i]) {
        const size_t z = (size_t)(offs[i] - pos < WC_ARTIFACT_ALIGN ? offs[i] - pos : WC_ARTIFACT_ALIGN);
        ok = fwrite(zeros, 1, z, file.f) == z;
        pos += z;
      }
      ok = ok && fwrite(h_containers[i], 1, (size_t)sizes[i], file.f) == sizes[i];
      pos += sizes[i];
    }
    ok = ok && fflush(file.f) == 0;
    if (!ok) {
      remove(tmp.c_str());
      return WC_E_IO;
    }
  }
  if (rename(tmp.c_str(), path) != 0) {
    remove(tmp.c_str());
    return WC_E_IO;
  }
  return WC_OK;
}

extern "C" int wc_artifact_count(const char* path, uint32_t* count) {
  if (!path || !count) return WC_E_ARG;
  File file(path, "rb");
  uint32_t n;
  uint64_t doff, fsize;
  int st = read_file_header(file, &n, &doff, &fsize);
  if (st != WC_OK) return st;
  // every container where the writer places it, and every byte between the
  // table and the data and between containers zero: with the CRCs, a change
  // to any byte of the file is then reported
  wc_artifact_info info;
  uint64_t gap_lo = kFileHeader + (uint64_t)kEntry * n, at = doff;
  uint8_t chunk[WC_ARTIFACT_ALIGN];
  for (uint32_t i = 0; i <= n; ++i) {
    uint64_t gap_hi = fsize;
    if (i < n) {
      st = read_entry(file, i, &info);
      if (st != WC_OK) return st;
      if (info.offset != at) return WC_E_CORRUPT;
      gap_hi = info.offset;
    }
    if (gap_hi < gap_lo || gap_hi - gap_lo >= WC_ARTIFACT_ALIGN) return WC_E_CORRUPT;
    const size_t len = (size_t)(gap_hi - gap_lo);
    if (len && !file.read_at(gap_lo, chunk, len)) return WC_E_CORRUPT;
    for (size_t k = 0; k < len; ++k)
      if (chunk[k]) return WC_E_CORRUPT;
    if (i < n) {
      gap_lo = info.offset + info.bytes;
      at = align_up(gap_lo);
    }
  }
  *count = n;
  return WC_OK;
}

extern "C" int wc_artifact_entry(const char* path, uint32_t i, wc_artifact_info* out) {
  if (!path || !out) return WC_E_ARG;
  File file(path, "rb");
  return read_entry(file, i, out);
}

extern "C" int wc_artifact_read(const char* path, uint32_t i, uint8_t* h_buf, size_t buf_bytes) {
  if (!path || !h_buf) return WC_E_ARG;
  File file(path, "rb");
  wc_artifact_info info;
  int st = read_entry(file, i, &info);
  if (st != WC_OK) return st;
  if (buf_bytes < info.bytes) return WC_E_SIZE;
  if (!file.read_at(info.offset, h_buf, (size_t)info.bytes)) return WC_E_CORRUPT;
  wc_header h;
  uint32_t crc[6];
  st = crcs_of(h_buf, (size_t)info.bytes, &h, crc);
  if (st != WC_OK) return WC_E_CORRUPT;
  uint64_t prod = 1;
  for (uint32_t k = 0; k < info.ndim; ++k) prod *= info.shape[k];
  if (h.total_bytes != info.bytes || h.layout != info.layout || h.n != prod) return WC_E_CORRUPT;
  for (int k = 0; k < 6; ++k)
    if (crc[k] != info.stream_crc[k]) return WC_E_CORRUPT;
  return WC_OK;
}
