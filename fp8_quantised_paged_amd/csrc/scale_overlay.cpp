// Revision-bound per-layer K/V scale file: written after offline calibration,
// read at start-up, failing closed on anything missing, foreign or invalid.
//
// Format (text, one record per line):
//   kvfp8-scale-overlay 1
//   revision <checkpoint revision, no whitespace>
//   layers <n>
//   <layer> <k_scale> <v_scale>      (n lines, layers 0 .. n-1 each once, any order)
// Scales are written as C99 hexadecimal floats, so a read returns the written
// fp32 values bit for bit.
#include <cerrno>
#include <cmath>
#include <cfloat>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kvfp8.h"

// Host-only code (no HIP calls): it also builds with a plain host compiler,
// which is how the sanitizer test builds it.
namespace kvfp8 {
void set_error(const char* msg);  // the library's thread-local error text
void clear_error();
}  // namespace kvfp8

#define KVFP8_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr const char* kMagic = "kvfp8-scale-overlay";
constexpr int kVersion = 1;
constexpr int kMaxLayers = 1 << 20;

// shares the library's thread-local error text through kvfp8_last_error
int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  kvfp8::set_error(buf);
  return status;
}

bool good_scale(float s) { return std::isfinite(s) && s >= FLT_MIN; }

bool good_revision(const char* r) {
  if (!r || !*r) return false;
  for (const char* p = r; *p; ++p)
    if (*p <= ' ' || *p == 0x7F) return false;
  return std::strlen(r) < 256;
}

// the whole line without its newline; false at end of file
bool read_line(FILE* f, std::string& line) {
  line.clear();
  int c;
  while ((c = std::fgetc(f)) != EOF && c != '\n') line.push_back((char)c);
  return !(c == EOF && line.empty());
}

// exact parse of one float token: the whole token must be consumed
bool parse_float(const char* tok, float* out) {
  if (!tok || !*tok) return false;
  char* end = nullptr;
  errno = 0;
  const float v = std::strtof(tok, &end);
  if (end == tok || *end != '\0') return false;
  *out = v;  // range errors leave Inf/0/subnormal, which the scale check rejects
  return true;
}

bool parse_int(const char* tok, long* out) {
  if (!tok || !*tok) return false;
  char* end = nullptr;
  errno = 0;
  const long v = std::strtol(tok, &end, 10);
  if (end == tok || *end != '\0' || errno == ERANGE) return false;
  *out = v;
  return true;
}

// splits on single spaces; false on any other whitespace or empty field
bool split(const std::string& line, std::vector<std::string>& out) {
  out.clear();
  std::string cur;
  for (char c : line) {
    if (c == ' ') {
      if (cur.empty()) return false;
      out.push_back(cur);
      cur.clear();
    } else if ((unsigned char)c < ' ' || c == 0x7F) {
      return false;
    } else {
      cur.push_back(c);
    }
  }
  if (cur.empty()) return false;
  out.push_back(cur);
  return true;
}

}  // namespace

KVFP8_API int32_t kvfp8_scale_overlay_write(const char* path, const char* revision, int32_t n_layers,
                                            const float* k_scales, const float* v_scales) {
  if (!path || !k_scales || !v_scales) return fail(KVFP8_INVALID_ARG, "null argument");
  if (!good_revision(revision))
    return fail(KVFP8_INVALID_ARG, "revision must be 1..255 printable characters without whitespace");
  if (n_layers <= 0 || n_layers > kMaxLayers) return fail(KVFP8_INVALID_ARG, "n_layers %d", n_layers);
  for (int32_t i = 0; i < n_layers; ++i)
    if (!good_scale(k_scales[i]) || !good_scale(v_scales[i]))
      return fail(KVFP8_BAD_SCALE, "layer %d: scales must be finite, positive and normal (got %g, %g)", i,
                  (double)k_scales[i], (double)v_scales[i]);
  const std::string tmp = std::string(path) + ".tmp";
  FILE* f = std::fopen(tmp.c_str(), "w");
  if (!f) return fail(KVFP8_INVALID_ARG, "cannot create %s: %s", tmp.c_str(), std::strerror(errno));
  bool ok = std::fprintf(f, "%s %d\nrevision %s\nlayers %d\n", kMagic, kVersion, revision, n_layers) > 0;
  for (int32_t i = 0; ok && i < n_layers; ++i)
    ok = std::fprintf(f, "%d %a %a\n", i, (double)k_scales[i], (double)v_scales[i]) > 0;
  ok = (std::fclose(f) == 0) && ok;
  if (!ok || std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return fail(KVFP8_INVALID_ARG, "cannot write %s", path);
  }
  kvfp8::clear_error();
  return KVFP8_OK;
}

KVFP8_API int32_t kvfp8_scale_overlay_read(const char* path, const char* revision, int32_t n_layers,
                                           float* k_scales, float* v_scales) {
  if (!path || !k_scales || !v_scales) return fail(KVFP8_INVALID_ARG, "null argument");
  if (!good_revision(revision)) return fail(KVFP8_INVALID_ARG, "invalid expected revision");
  if (n_layers <= 0 || n_layers > kMaxLayers) return fail(KVFP8_INVALID_ARG, "n_layers %d", n_layers);
  FILE* f = std::fopen(path, "r");
  if (!f) return fail(KVFP8_INVALID_ARG, "scale overlay %s is missing: %s", path, std::strerror(errno));
  std::string line;
  std::vector<std::string> tok;
  std::vector<float> k((size_t)n_layers), v((size_t)n_layers);
  std::vector<char> seen((size_t)n_layers, 0);
  int32_t status = KVFP8_OK;
  long val = 0;
  // header
  if (!read_line(f, line) || !split(line, tok) || tok.size() != 2 || tok[0] != kMagic ||
      !parse_int(tok[1].c_str(), &val) || val != kVersion) {
    status = fail(KVFP8_INVALID_ARG, "%s: not a version-%d scale overlay", path, kVersion);
  } else if (!read_line(f, line) || !split(line, tok) || tok.size() != 2 || tok[0] != "revision") {
    status = fail(KVFP8_INVALID_ARG, "%s: missing revision line", path);
  } else if (tok[1] != revision) {
    status = fail(KVFP8_INVALID_ARG, "%s: calibrated for revision %s, not %s", path, tok[1].c_str(), revision);
  } else if (!read_line(f, line) || !split(line, tok) || tok.size() != 2 || tok[0] != "layers" ||
             !parse_int(tok[1].c_str(), &val)) {
    status = fail(KVFP8_INVALID_ARG, "%s: missing layers line", path);
  } else if (val != n_layers) {
    status = fail(KVFP8_INVALID_ARG, "%s: holds %ld layers, %d expected", path, val, n_layers);
  }
  // records
  int32_t count = 0;
  while (status == KVFP8_OK && read_line(f, line)) {
    float ks = 0.0f, vs = 0.0f;
    if (!split(line, tok) || tok.size() != 3 || !parse_int(tok[0].c_str(), &val) ||
        !parse_float(tok[1].c_str(), &ks) || !parse_float(tok[2].c_str(), &vs)) {
      status = fail(KVFP8_INVALID_ARG, "%s: malformed record '%s'", path, line.c_str());
    } else if (val < 0 || val >= n_layers) {
      status = fail(KVFP8_INVALID_ARG, "%s: layer %ld out of range", path, val);
    } else if (seen[(size_t)val]) {
      status = fail(KVFP8_INVALID_ARG, "%s: layer %ld appears twice", path, val);
    } else if (!good_scale(ks) || !good_scale(vs)) {
      status = fail(KVFP8_BAD_SCALE, "%s: layer %ld scales must be finite, positive and normal (got %g, %g)",
                    path, val, (double)ks, (double)vs);
    } else {
      seen[(size_t)val] = 1;
      k[(size_t)val] = ks;
      v[(size_t)val] = vs;
      ++count;
    }
  }
  std::fclose(f);
  if (status == KVFP8_OK && count != n_layers) {
    int32_t missing = 0;
    while (missing < n_layers && seen[(size_t)missing]) ++missing;
    status = fail(KVFP8_INVALID_ARG, "%s: layer %d has no scales (%d of %d present)", path, missing, count,
                  n_layers);
  }
  if (status != KVFP8_OK) return status;  // outputs are written only on success
  std::memcpy(k_scales, k.data(), sizeof(float) * (size_t)n_layers);
  std::memcpy(v_scales, v.data(), sizeof(float) * (size_t)n_layers);
  kvfp8::clear_error();
  return KVFP8_OK;
}
