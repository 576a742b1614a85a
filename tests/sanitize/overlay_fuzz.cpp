// Host-only robustness check of the scale-overlay reader and writer, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize_host.py.
// A valid 24-layer file is written, then thousands of seeded mutations of it
// (byte flips, deletions, duplications, insertions, truncations, long lines,
// extreme numbers) are read back. Every read must return OK, INVALID_ARG or
// BAD_SCALE; a failed read must leave the outputs untouched; a successful read
// must return finite, positive, normal scales for every layer. Any memory or
// undefined-behaviour error aborts the run (non-zero exit).
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kvfp8.h"

// the library's error-text hooks (defined in api.cpp, not linked here)
namespace kvfp8 {
static char g_text[512];
void set_error(const char* msg) { std::snprintf(g_text, sizeof(g_text), "%s", msg); }
void clear_error() { g_text[0] = '\0'; }
}  // namespace kvfp8

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
size_t below(size_t n) { return n ? (size_t)(next() % n) : 0; }

std::string slurp(const char* path) {
  std::string s;
  FILE* f = std::fopen(path, "rb");
  if (!f) return s;
  int c;
  while ((c = std::fgetc(f)) != EOF) s.push_back((char)c);
  std::fclose(f);
  return s;
}

void spit(const char* path, const std::string& s) {
  FILE* f = std::fopen(path, "wb");
  if (!f) return;
  std::fwrite(s.data(), 1, s.size(), f);
  std::fclose(f);
}

const char* kTokens[] = {"0x1p+200", "nan", "-inf", "inf", "0x1p-140", "-0x1p-3", "0", "1e39",
                         "99999999999999999999", "-1", "24", "23", "layers", "revision", "\t", "  ",
                         "kvfp8-scale-overlay 1", "0x1.8p-1 0x1.8p-1", "\n", "\r\n"};

std::string mutate(const std::string& base) {
  std::string s = base;
  const int n = 1 + (int)below(4);
  for (int m = 0; m < n; ++m) {
    const size_t at = below(s.size() + 1);
    switch (below(8)) {
      case 0:  // flip a byte
        if (!s.empty()) s[below(s.size())] ^= (char)(1u << below(8));
        break;
      case 1:  // delete a range
        if (!s.empty()) s.erase(at > 0 ? at - 1 : 0, 1 + below(16));
        break;
      case 2: {  // duplicate a range
        const size_t from = below(s.size() + 1);
        s.insert(at, s.substr(from, below(64)));
        break;
      }
      case 3:  // insert a token
        s.insert(at, kTokens[below(sizeof(kTokens) / sizeof(kTokens[0]))]);
        break;
      case 4:  // truncate
        s.resize(below(s.size() + 1));
        break;
      case 5:  // a very long line
        s.insert(at, std::string(1000 + below(20000), (char)('0' + below(10))));
        break;
      case 6:  // random bytes, NUL included
        for (size_t k = below(8) + 1; k > 0; --k) s.insert(s.begin() + (long)below(s.size() + 1), (char)below(256));
        break;
      default:  // swap two lines' worth of text
        if (s.size() > 2) std::swap(s[below(s.size())], s[below(s.size())]);
        break;
    }
  }
  return s;
}

}  // namespace

int main(int argc, char** argv) {
  const char* dir = argc > 1 ? argv[1] : "/tmp";
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 3000;
  const std::string good = std::string(dir) + "/overlay_good.txt";
  const std::string bad = std::string(dir) + "/overlay_fuzz.txt";
  const int32_t L = 24;
  std::vector<float> ks(L), vs(L);
  for (int i = 0; i < L; ++i) {
    ks[(size_t)i] = std::ldexp(1.0f + (float)i / 32.0f, -7 + i % 5);
    vs[(size_t)i] = std::ldexp(1.5f - (float)i / 64.0f, -6 + i % 3);
  }
  if (kvfp8_scale_overlay_write(good.c_str(), "rev-abc123", L, ks.data(), vs.data()) != KVFP8_OK) return 2;
  std::vector<float> rk(L), rv(L);
  if (kvfp8_scale_overlay_read(good.c_str(), "rev-abc123", L, rk.data(), rv.data()) != KVFP8_OK) return 3;
  if (std::memcmp(rk.data(), ks.data(), sizeof(float) * L) || std::memcmp(rv.data(), vs.data(), sizeof(float) * L))
    return 4;
  const std::string base = slurp(good.c_str());
  int ok = 0, invalid = 0, badscale = 0;
  for (int r = 0; r < rounds; ++r) {
    spit(bad.c_str(), r % 50 == 1 ? base : mutate(base));  // some untouched copies must read back
    const float sentinel = -12345.0f;
    std::vector<float> ok_k(L, sentinel), ok_v(L, sentinel);
    const char* rev = (r % 17 == 0) ? "rev-other" : "rev-abc123";
    const int32_t layers = (r % 23 == 0) ? L - 1 : L;
    const int32_t st = kvfp8_scale_overlay_read(bad.c_str(), rev, layers, ok_k.data(), ok_v.data());
    if (st == KVFP8_OK) {
      ++ok;
      for (int i = 0; i < layers; ++i) {
        const float a = ok_k[(size_t)i], b = ok_v[(size_t)i];
        if (!(std::isfinite(a) && a >= FLT_MIN && std::isfinite(b) && b >= FLT_MIN)) return 5;
      }
    } else if (st == KVFP8_INVALID_ARG || st == KVFP8_BAD_SCALE) {
      (st == KVFP8_INVALID_ARG ? invalid : badscale)++;
      for (int i = 0; i < L; ++i)
        if (ok_k[(size_t)i] != sentinel || ok_v[(size_t)i] != sentinel) return 6;  // touched on failure
    } else {
      return 7;
    }
  }
  std::remove(good.c_str());
  std::remove(bad.c_str());
  std::printf("overlay fuzz: %d reads ok, %d invalid, %d bad scale\n", ok, invalid, badscale);
  return (invalid > 0 && ok > 0) ? 0 : 8;  // the mutations must exercise both outcomes
}
