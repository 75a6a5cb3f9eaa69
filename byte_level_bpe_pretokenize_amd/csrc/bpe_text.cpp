// bpe_text.cpp -- the text form of a merge table and a vocabulary, parsed on
// the host into the integer form that bpe_load_merges takes.
//
// "Tokenization LLM: details of building an inference engine in C++", section
// "Byte-level encoding": a table that maps each of the 256 byte values to a
// printable character, so that merges and vocabularies can be stored as text
// (the byte 0xF0 prints as U+00F0); section "Vocabulary lookup": the merged
// symbols become IDs through the vocabulary (" world" is stored as
// "Ġworld").  Reading of the open points: the 188 bytes 0x21-0x7E,
// 0xA1-0xAC and 0xAE-0xFF print as the code point of the same value, the
// other 68 bytes as U+0100, U+0101, ... in increasing byte order (so 0x20 is
// U+0120); a merges file is one merge per line, "left right" with a single
// space, in rank order, after an optional first line starting with
// "#version"; each operand must be a byte or the result of an earlier line,
// and no two lines may give the same byte string; a vocabulary is a JSON
// object from token text to ID.
#include <stdint.h>
#include <string.h>

#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/bpe.h"

namespace {

// Code point of byte b in the printable map, and the byte of each code point
// (-1 where none).
struct PrintMap {
  int32_t cp[256];
  int32_t byte_of[0x144];
  PrintMap() {
    for (int i = 0; i < 0x144; ++i) byte_of[i] = -1;
    int n = 0;
    for (int b = 0; b < 256; ++b) {
      const bool same = (b >= 0x21 && b <= 0x7E) || (b >= 0xA1 && b <= 0xAC) || (b >= 0xAE);
      cp[b] = same ? b : 0x100 + n++;
      byte_of[cp[b]] = b;
    }
  }
};

const PrintMap &print_map() {
  static const PrintMap m;
  return m;
}

// Next code point of UTF-8 text s[*i .. n), or -1 for a malformed sequence.
int32_t utf8_next(const unsigned char *s, int64_t n, int64_t *i) {
  const unsigned c = s[*i];
  int len = c < 0x80 ? 1 : (c >> 5) == 6 ? 2 : (c >> 4) == 14 ? 3 : (c >> 3) == 30 ? 4 : 0;
  if (len == 0 || *i + len > n) return -1;
  int32_t cp = len == 1 ? (int32_t)c : (int32_t)(c & (0x7F >> len));
  for (int k = 1; k < len; ++k) {
    const unsigned x = s[*i + k];
    if ((x >> 6) != 2) return -1;
    cp = (cp << 6) | (int32_t)(x & 0x3F);
  }
  *i += len;
  return cp;
}

// Bytes of printable text (code points of the print map), false if some code
// point is not in it.
bool text_bytes(const int32_t *cps, size_t n, std::string *out) {
  const PrintMap &m = print_map();
  out->clear();
  for (size_t k = 0; k < n; ++k) {
    if (cps[k] < 0 || cps[k] >= 0x144 || m.byte_of[cps[k]] < 0) return false;
    out->push_back((char)m.byte_of[cps[k]]);
  }
  return true;
}

bool utf8_bytes(const unsigned char *s, int64_t n, std::string *out) {
  std::vector<int32_t> cps;
  for (int64_t i = 0; i < n;) {
    const int32_t cp = utf8_next(s, n, &i);
    if (cp < 0) return false;
    cps.push_back(cp);
  }
  return text_bytes(cps.data(), cps.size(), out);
}

// Byte expansion of every symbol of a table (0..255 the bytes), or false if
// an operand is out of range or depends on itself.
bool expansions(const int32_t *merges, int64_t R, std::vector<std::string> *exp) {
  const int64_t V = 256 + R;
  exp->assign((size_t)V, std::string());
  std::vector<char> done((size_t)V, 0);
  for (int b = 0; b < 256; ++b) {
    (*exp)[(size_t)b] = std::string(1, (char)b);
    done[(size_t)b] = 1;
  }
  for (bool progress = true; progress;) {
    progress = false;
    for (int64_t r = 0; r < R; ++r) {
      const int64_t s = 256 + r, l = merges[2 * r], rr = merges[2 * r + 1];
      if (done[(size_t)s]) continue;
      if (l < 0 || l >= V || rr < 0 || rr >= V) return false;
      if (!done[(size_t)l] || !done[(size_t)rr]) continue;
      (*exp)[(size_t)s] = (*exp)[(size_t)l] + (*exp)[(size_t)rr];
      done[(size_t)s] = 1;
      progress = true;
    }
  }
  for (int64_t s = 0; s < V; ++s)
    if (!done[(size_t)s]) return false;
  return true;
}

// ---- a minimal JSON reader for an object of string keys and integer values ----
struct Json {
  const unsigned char *s;
  int64_t n, i = 0;
  void ws() {
    while (i < n && (s[i] == ' ' || s[i] == '\t' || s[i] == '\n' || s[i] == '\r')) ++i;
  }
  bool hex4(int32_t *v) {
    if (i + 4 > n) return false;
    int32_t x = 0;
    for (int k = 0; k < 4; ++k) {
      const unsigned c = s[i + k];
      const int d = c >= '0' && c <= '9' ? (int)c - '0'
                    : c >= 'a' && c <= 'f' ? (int)c - 'a' + 10
                    : c >= 'A' && c <= 'F' ? (int)c - 'A' + 10
                                           : -1;
      if (d < 0) return false;
      x = x * 16 + d;
    }
    i += 4;
    *v = x;
    return true;
  }
  // a string's code points
  bool str(std::vector<int32_t> *cps) {
    cps->clear();
    if (i >= n || s[i] != '"') return false;
    ++i;
    while (i < n && s[i] != '"') {
      if (s[i] == '\\') {
        if (++i >= n) return false;
        const unsigned e = s[i++];
        int32_t cp;
        switch (e) {
          case '"': cp = '"'; break;
          case '\\': cp = '\\'; break;
          case '/': cp = '/'; break;
          case 'b': cp = 8; break;
          case 'f': cp = 12; break;
          case 'n': cp = 10; break;
          case 'r': cp = 13; break;
          case 't': cp = 9; break;
          case 'u': {
            if (!hex4(&cp)) return false;
            if (cp >= 0xD800 && cp < 0xDC00) {  // a surrogate pair
              int32_t lo;
              if (i + 2 > n || s[i] != '\\' || s[i + 1] != 'u') return false;
              i += 2;
              if (!hex4(&lo) || lo < 0xDC00 || lo >= 0xE000) return false;
              cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
            }
            break;
          }
          default: return false;
        }
        cps->push_back(cp);
      } else {
        const int32_t cp = utf8_next(s, n, &i);
        if (cp < 0) return false;
        cps->push_back(cp);
      }
    }
    if (i >= n) return false;
    ++i;
    return true;
  }
  bool integer(int64_t *v) {
    bool neg = false;
    if (i < n && s[i] == '-') {
      neg = true;
      ++i;
    }
    if (i >= n || s[i] < '0' || s[i] > '9') return false;
    int64_t x = 0;
    while (i < n && s[i] >= '0' && s[i] <= '9') {
      x = x * 10 + (s[i++] - '0');
      if (x > ((int64_t)1 << 40)) return false;
    }
    *v = neg ? -x : x;
    return true;
  }
};

}  // namespace

extern "C" {

int bpe_parse_merges_text(const char *text, int64_t text_len, int32_t *merges_out,
                          int64_t max_merges, int64_t *n_merges) {
  if (!text || text_len < 0 || max_merges < 0 || !n_merges || (max_merges > 0 && !merges_out))
    return BPE_EINVAL;
  const unsigned char *s = (const unsigned char *)text;
  std::unordered_map<std::string, int32_t> sym;
  for (int b = 0; b < 256; ++b) sym.emplace(std::string(1, (char)b), b);
  int64_t R = 0;
  std::string lb, rb;
  bool first = true;
  for (int64_t i = 0; i < text_len;) {
    int64_t e = i;
    while (e < text_len && s[e] != '\n') ++e;
    int64_t end = e;
    if (end > i && s[end - 1] == '\r') --end;
    const bool header = first && end - i >= 8 && memcmp(s + i, "#version", 8) == 0;
    first = false;
    if (end > i && !header) {
      int64_t sp = -1;
      for (int64_t k = i; k < end; ++k)
        if (s[k] == ' ') {
          if (sp >= 0) return BPE_EFORMAT;
          sp = k;
        }
      if (sp <= i || sp + 1 >= end) return BPE_EFORMAT;
      if (!utf8_bytes(s + i, sp - i, &lb) || !utf8_bytes(s + sp + 1, end - sp - 1, &rb))
        return BPE_EFORMAT;
      const auto l = sym.find(lb), r = sym.find(rb);
      if (l == sym.end() || r == sym.end()) return BPE_EMERGES;
      if (R >= BPE_MAX_MERGES) return BPE_EMERGES;
      if (R >= max_merges) return BPE_EINVAL;
      if (!sym.emplace(lb + rb, (int32_t)(256 + R)).second) return BPE_EMERGES;
      merges_out[2 * R] = l->second;
      merges_out[2 * R + 1] = r->second;
      ++R;
    }
    i = e + 1;
  }
  *n_merges = R;
  return BPE_OK;
}

int bpe_parse_vocab_json(const char *json, int64_t json_len, const int32_t *merges,
                         int64_t n_merges, int32_t *id_map_out) {
  if (!json || json_len < 0 || n_merges < 0 || n_merges > BPE_MAX_MERGES || !id_map_out ||
      (n_merges > 0 && !merges))
    return BPE_EINVAL;
  std::vector<std::string> exp;
  if (!expansions(merges, n_merges, &exp)) return BPE_EMERGES;
  std::unordered_map<std::string, int64_t> id;
  Json j{(const unsigned char *)json, json_len};
  std::vector<int32_t> cps;
  std::string key;
  j.ws();
  if (j.i >= j.n || j.s[j.i] != '{') return BPE_EFORMAT;
  ++j.i;
  j.ws();
  if (j.i < j.n && j.s[j.i] == '}') {
    ++j.i;
  } else {
    for (;;) {
      j.ws();
      if (!j.str(&cps)) return BPE_EFORMAT;
      j.ws();
      if (j.i >= j.n || j.s[j.i] != ':') return BPE_EFORMAT;
      ++j.i;
      j.ws();
      int64_t v;
      if (!j.integer(&v)) return BPE_EFORMAT;
      // text outside the print map (a marker such as a reserved ID's name
      // may be) names no symbol
      if (text_bytes(cps.data(), cps.size(), &key)) id[key] = v;
      j.ws();
      if (j.i < j.n && j.s[j.i] == ',') {
        ++j.i;
        continue;
      }
      if (j.i < j.n && j.s[j.i] == '}') {
        ++j.i;
        break;
      }
      return BPE_EFORMAT;
    }
  }
  j.ws();
  if (j.i != j.n) return BPE_EFORMAT;
  for (size_t v = 0; v < exp.size(); ++v) {
    const auto f = id.find(exp[v]);
    if (f == id.end() || f->second < 0 || f->second > BPE_MAX_ID) return BPE_EIDMAP;
    id_map_out[v] = (int32_t)f->second;
  }
  return BPE_OK;
}

}  // extern "C"
