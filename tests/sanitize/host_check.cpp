// host_check.cpp — drives the library's host-only code under AddressSanitizer
// and UndefinedBehaviorSanitizer: the container header check (validate_header)
// and the serialized artifact (wc_artifact.hip: CRC-32, per-region container
// CRCs, writer and readers).  Test infrastructure, built host-only and run by
// tests/test_sanitizers.py; containers come from the CPU oracle.
//
// Checks: the CRC against a bit-at-a-time CRC-32 written here; the header
// check against the oracle's own header reader on every single-bit change of
// every test container's header and on random headers (both must accept
// exactly the same headers); artifact round trips; and every byte of an
// artifact file changed in turn, each of which the readers must report as
// WC_E_CORRUPT.  Usage: host_check DIR (a scratch directory for the files).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "wc_common.h"
#include "wc_oracle.h"

namespace {

int failures = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                        \
      fputc('\n', stderr);                                 \
      ++failures;                                          \
    }                                                      \
  } while (0)

// splitmix64: the seeded bit source of the inputs (no part of the method)
uint64_t mix_state = 77;
uint64_t next64() {
  uint64_t z = (mix_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// CRC-32 one bit at a time (reflected, polynomial 0xEDB88320)
uint32_t crc_bitwise(const uint8_t* p, size_t n) {
  uint32_t c = 0xFFFFFFFFu;
  for (size_t i = 0; i < n; ++i) {
    c ^= p[i];
    for (int k = 0; k < 8; ++k) c = (c >> 1) ^ (0xEDB88320u & (0u - (c & 1u)));
  }
  return ~c;
}

std::vector<uint16_t> weights(uint64_t n, unsigned rare, bool uniform) {
  std::vector<uint16_t> w(n);
  for (uint64_t i = 0; i < n; ++i) {
    const uint64_t r = next64();
    if (uniform) {
      w[i] = (uint16_t)r;
      continue;
    }
    uint32_t ex = 121u + (uint32_t)((r >> 8) % 6u);
    if ((r >> 20) % 1024u < rare) ex = (uint32_t)((r >> 32) & 0xFFu);
    w[i] = (uint16_t)((uint32_t)(r >> 63) << 15 | ex << 7 | (uint32_t)(r & 0x7Fu));
  }
  return w;
}

struct Item {
  std::string name;
  uint32_t ndim;
  uint64_t shape[4];
  std::vector<uint16_t> src;
  std::vector<uint8_t> c;
};

Item make(const char* name, int layout, int flags, std::vector<uint64_t> shape, unsigned rare,
          bool uniform) {
  Item it;
  it.name = name;
  it.ndim = (uint32_t)shape.size();
  uint64_t n = 1;
  for (int k = 0; k < 4; ++k) {
    it.shape[k] = k < (int)shape.size() ? shape[k] : 0;
    if (k < (int)shape.size()) n *= shape[k];
  }
  it.src = weights(n, rare, uniform);
  it.c.resize(1024 + 16 * n);
  uint64_t size = 0;
  const int rc = orc_encode_flags(layout, flags, it.src.data(), n, it.c.data(), it.c.size(), &size);
  CHECK(rc == ORC_OK, "oracle encode %s: %d", name, rc);
  it.c.resize(size);
  return it;
}

bool header_ok_oracle(const uint8_t* h) {
  int layout, n_dict;
  uint64_t n, n_esc, off[6];
  uint16_t dict[16];
  return orc_header_info(h, 1ull << 40, &layout, &n_dict, &n, &n_esc, dict, off) == ORC_OK;
}

bool header_ok_library(const uint8_t* h) {
  wc_header hh;
  memcpy(&hh, h, sizeof hh);
  return wc::validate_header(&hh) == WC_OK;
}

// Reads every entry of the artifact as a user would: count, then each entry's
// metadata and container.  Returns the first error code, or WC_OK.
int read_all(const char* path, const std::vector<Item>* want) {
  uint32_t count = 0;
  int st = wc_artifact_count(path, &count);
  if (st != WC_OK) return st;
  for (uint32_t i = 0; i < count; ++i) {
    wc_artifact_info info;
    st = wc_artifact_entry(path, i, &info);
    if (st != WC_OK) return st;
    std::vector<uint8_t> buf(info.bytes);
    st = wc_artifact_read(path, i, buf.data(), buf.size());
    if (st != WC_OK) return st;
    // the delivered weights against the source's CRC: the reader's last check
    uint64_t n = 1;
    for (uint32_t k = 0; k < info.ndim; ++k) n *= info.shape[k];
    std::vector<uint16_t> dec(n ? n : 1);
    if (orc_decode(buf.data(), buf.size(), dec.data(), n) != ORC_OK) return WC_E_CORRUPT;
    if (crc_bitwise((const uint8_t*)dec.data(), 2 * n) != info.src_crc) return WC_E_CORRUPT;
    if (want && (i >= want->size() || buf != (*want)[i].c)) return -100;
  }
  if (want && count != want->size()) return -101;
  return WC_OK;
}

int write_artifact(const char* path, const std::vector<Item>& items) {
  std::vector<const char*> names;
  std::vector<uint32_t> ndims, crcs;
  std::vector<uint64_t> shapes, bytes;
  std::vector<const uint8_t*> ptrs;
  for (const Item& it : items) {
    names.push_back(it.name.c_str());
    ndims.push_back(it.ndim);
    for (int k = 0; k < 4; ++k) shapes.push_back(it.shape[k]);
    ptrs.push_back(it.c.data());
    bytes.push_back(it.c.size());
    crcs.push_back(crc_bitwise((const uint8_t*)it.src.data(), 2 * it.src.size()));
  }
  return wc_artifact_write(path, (uint32_t)items.size(), names.data(), ndims.data(), shapes.data(),
                           ptrs.data(), bytes.data(), crcs.data());
}

void flip_byte(const char* path, uint64_t off, uint8_t mask) {
  FILE* f = fopen(path, "r+b");
  CHECK(f != nullptr, "open %s", path);
  if (!f) return;
  uint8_t b = 0;
  fseeko(f, (off_t)off, SEEK_SET);
  CHECK(fread(&b, 1, 1, f) == 1, "read byte %llu", (unsigned long long)off);
  b ^= mask;
  fseeko(f, (off_t)off, SEEK_SET);
  CHECK(fwrite(&b, 1, 1, f) == 1, "write byte %llu", (unsigned long long)off);
  fclose(f);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: host_check DIR\n");
    return 2;
  }
  const std::string dir = argv[1];

  // ---- CRC-32
  CHECK(wc_crc32(0, "123456789", 9) == 0xCBF43926u, "check value");
  for (int t = 0; t < 300; ++t) {
    std::vector<uint8_t> b(1 + t * 7);
    for (auto& x : b) x = (uint8_t)next64();
    const size_t lo = (size_t)t % 9, len = b.size() - lo;
    CHECK(wc_crc32(0, b.data() + lo, len) == crc_bitwise(b.data() + lo, len), "crc length %zu", len);
    const size_t cut = len / 3;
    CHECK(wc_crc32(wc_crc32(0, b.data() + lo, cut), b.data() + lo + cut, len - cut) ==
              crc_bitwise(b.data() + lo, len),
          "continued crc");
  }
  printf("crc: ok\n");

  // ---- containers from the oracle
  std::vector<Item> items;
  items.push_back(make("bs.3000", WC_LAYOUT_BYTESPLIT, 0, {3, 1000}, 40, false));
  items.push_back(make("k15.compact", WC_LAYOUT_K15, WC_FLAG_COMPACT, {2500}, 40, false));
  items.push_back(make("bs.compact.uniform", WC_LAYOUT_BYTESPLIT, WC_FLAG_COMPACT, {10, 70}, 0, true));
  items.push_back(make("raw", WC_LAYOUT_RAW, 0, {7, 100}, 0, true));
  items.push_back(make("k15.4d", WC_LAYOUT_K15, 0, {2, 3, 5, 137}, 0, false));
  items.push_back(make("empty", WC_LAYOUT_BYTESPLIT, 0, {0}, 0, false));

  // ---- header check: the library's and the oracle's accept the same headers
  uint64_t flips = 0, accepted = 0;
  for (const Item& it : items) {
    CHECK(header_ok_library(it.c.data()) && header_ok_oracle(it.c.data()), "valid header %s",
          it.name.c_str());
    uint32_t crc[6];
    CHECK(wc_container_crcs(it.c.data(), it.c.size(), crc) == WC_OK, "crcs %s", it.name.c_str());
    wc_header h;
    memcpy(&h, it.c.data(), sizeof h);
    const uint64_t b[7] = {0, 128, h.off_raw, h.off_esc_pos, h.off_esc_sym, h.off_esc_idx, h.total_bytes};
    for (int k = 0; k < 6; ++k)
      CHECK(crc[k] == crc_bitwise(it.c.data() + b[k], (size_t)(b[k + 1] - b[k])), "region %d of %s", k,
            it.name.c_str());
    // one byte short: a header alone is short of its 128 bytes, else of total_bytes
    // (a copy of exactly that size, so a read past it is a sanitizer report)
    const std::vector<uint8_t> shortc(it.c.begin(), it.c.end() - 1);
    CHECK(wc_container_crcs(shortc.data(), shortc.size(), crc) ==
              (shortc.size() < 128 ? WC_E_CORRUPT : WC_E_SIZE),
          "short container %s", it.name.c_str());
    for (int bit = 0; bit < 128 * 8; ++bit) {
      uint8_t hb[128];
      memcpy(hb, it.c.data(), 128);
      hb[bit / 8] ^= (uint8_t)(1u << (bit % 8));
      const bool lib = header_ok_library(hb), orc = header_ok_oracle(hb);
      CHECK(lib == orc, "%s bit %d: library %d oracle %d", it.name.c_str(), bit, lib, orc);
      ++flips;
      accepted += lib;
    }
  }
  uint64_t random_ok = 0;
  for (int t = 0; t < 50000; ++t) {
    uint8_t hb[128];
    for (auto& x : hb) x = (uint8_t)next64();
    // a valid magic, version and layout, then random fields; every few, the
    // reserved tail and unused dictionary slots zeroed so deeper checks run
    memcpy(hb, "WC16", 4);
    hb[4] = 2;
    hb[5] = 0;
    hb[6] = (uint8_t)(t % 3);
    if (t % 2) {
      hb[7] = (uint8_t)(t % 16);
      memset(hb + 9 + 3, 0, 4);   // n below 2^32
      memset(hb + 16 + 3, 0, 5);  // n_esc small
    }
    if (t % 4 == 1) memset(hb + 104, 0, 24);
    if (t % 8 == 3) {
      // offsets that fit the fields, so the dictionary checks decide
      wc_header h;
      memcpy(&h, hb, sizeof h);
      if (h.n < (1ull << 32) && h.n_esc <= h.n) {
        h.n_dict = (uint8_t)(t / 8 % 16);
        for (int k = h.n_dict; k < 16; ++k) h.dict[k] = 0;
        for (int k = 0; k < h.n_dict; ++k) h.dict[k] = (uint16_t)(next64() % 520u);
        h.flags = h.layout == WC_LAYOUT_RAW ? 0 : (uint8_t)(t / 128 % 2);
        if (h.layout == WC_LAYOUT_RAW) h.n_dict = 0, h.n_esc = 0, memset(h.dict, 0, sizeof h.dict);
        memset(h.reserved, 0, sizeof h.reserved);
        const wc::Geometry g = wc::geometry(h.layout, h.n, h.n_esc, h.flags);
        h.off_codes = g.off_codes;
        h.off_raw = g.off_raw;
        h.off_esc_pos = g.off_esc_pos;
        h.off_esc_sym = g.off_esc_sym;
        h.off_esc_idx = g.off_esc_idx;
        h.total_bytes = g.total;
        memcpy(hb, &h, sizeof h);
      }
    }
    const bool lib = header_ok_library(hb);
    CHECK(lib == header_ok_oracle(hb), "random header %d", t);
    random_ok += lib;
  }
  printf("header check: %llu single-bit changes (%llu still valid), 50000 random headers "
         "(%llu valid)\n",
         (unsigned long long)flips, (unsigned long long)accepted, (unsigned long long)random_ok);

  // ---- artifact round trip
  const std::string path = dir + "/a.wca";
  CHECK(write_artifact(path.c_str(), items) == WC_OK, "write");
  CHECK(read_all(path.c_str(), &items) == WC_OK, "round trip");
  FILE* f = fopen(path.c_str(), "rb");
  fseeko(f, 0, SEEK_END);
  const uint64_t fsize = (uint64_t)ftello(f);
  fclose(f);

  // ---- every byte of the file changed in turn: always reported as corrupt
  uint64_t undetected = 0;
  for (uint64_t off = 0; off < fsize; ++off) {
    const uint8_t mask = (uint8_t)(1u << (off % 8));
    flip_byte(path.c_str(), off, mask);
    const int st = read_all(path.c_str(), nullptr);
    if (st != WC_E_CORRUPT) {
      ++undetected;
      CHECK(false, "byte %llu changed: read gives %d", (unsigned long long)off, st);
    }
    flip_byte(path.c_str(), off, mask);
  }
  CHECK(read_all(path.c_str(), &items) == WC_OK, "restored file");
  printf("artifact: %llu bytes, each changed in turn, %llu undetected\n", (unsigned long long)fsize,
         (unsigned long long)undetected);

  // ---- truncated, extended and missing files
  {
    std::vector<uint8_t> all(fsize);
    f = fopen(path.c_str(), "rb");
    CHECK(fread(all.data(), 1, fsize, f) == fsize, "read file");
    fclose(f);
    const std::string bad = dir + "/b.wca";
    for (uint64_t cut : {fsize - 1, fsize / 2, (uint64_t)4096, (uint64_t)63, (uint64_t)0}) {
      f = fopen(bad.c_str(), "wb");
      if (cut) fwrite(all.data(), 1, cut, f);
      fclose(f);
      CHECK(read_all(bad.c_str(), nullptr) == WC_E_CORRUPT, "cut at %llu", (unsigned long long)cut);
    }
    f = fopen(bad.c_str(), "wb");
    fwrite(all.data(), 1, fsize, f);
    fputc(0, f);
    fclose(f);
    CHECK(read_all(bad.c_str(), nullptr) == WC_E_CORRUPT, "byte appended");
    CHECK(read_all((dir + "/missing.wca").c_str(), nullptr) == WC_E_IO, "missing file");
  }

  // ---- writer argument checks: nothing is written on a refusal
  {
    const std::string p = dir + "/w.wca";
    remove(p.c_str());
    std::vector<Item> one(items.begin(), items.begin() + 1);
    one[0].name = std::string(96, 'x');
    CHECK(write_artifact(p.c_str(), one) == WC_E_ARG, "long name");
    one[0].name = "ok";
    one[0].shape[1] = 999;
    CHECK(write_artifact(p.c_str(), one) == WC_E_ARG, "shape product");
    one[0].shape[1] = 1000;
    one[0].c[6] = 7;  // layout byte
    CHECK(write_artifact(p.c_str(), one) == WC_E_CORRUPT, "bad container");
    f = fopen(p.c_str(), "rb");
    CHECK(f == nullptr, "refused write left a file");
    if (f) fclose(f);
    std::vector<Item> none;
    CHECK(write_artifact(p.c_str(), none) == WC_OK && read_all(p.c_str(), &none) == WC_OK, "empty artifact");
  }

  printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
