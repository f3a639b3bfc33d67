// Checkpoint loading (host only): config.json of a Qwen3 model into a dec_config, and a
// model.safetensors file into the library's weights blob.
//
// Sources: "Candle model runner" section 2.3 (the model directory: what the engine cannot run is
// refused at load with a message; the safetensors layout, ranges counted from the data buffer
// and tiling it exactly; F16 / BF16 widening) and section 2.5 (int4 weights, loaded from an
// int4 file or quantised at load); "A real model in our own decoder" (the Qwen3 settings, the
// reader that trusts nothing in the file, the tied matrix stored twice).
//
// The rules this reader applies, in the order it applies them:
//   F1  the file holds at least the 8-byte little-endian header size N;
//   F2  2 <= N <= kMaxHeader and the header ends inside the file;
//   F3  the header is one JSON object without a repeated key at any depth;
//   F4  "__metadata__", when present, maps names to strings; "quant" there names the int4
//       format of the file ("int4-g32-sym"), any other value is refused;
//   F5  every other entry names a tensor: dtype F32, F16, BF16, U8 (int4 values) or any other
//       (refused as unsupported), a shape of non-negative integers, and data_offsets
//       [begin, end] with begin <= end;
//   F6  end - begin is the element count times the element size;
//   F7  the payload (the bytes after the header) is tiled by the ranges: every range inside it,
//       no two ranges sharing a byte, and their lengths adding up to the payload's size;
//   F8  the names are Hugging Face's Qwen3 names and nothing else: every expected tensor is
//       present with its expected shape, and no other tensor is;
//   F9  an lm_head tensor, when present, holds the embedding's values.
// A matrix is stored as "<name>.weight" (F32 / F16 / BF16) or, in an int4 file, as
// "<name>.qweight" (U8 [out][in/2], the runner's nibble order) and "<name>.scales" (F16
// [out][in/32]). Gains are always "<name>.weight".
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "dec.h"

namespace {

// ---- a small JSON reader (objects keep their key order; a repeated key is an error) ----------
struct Json {
  enum Type { NUL, BOOL, NUM, STR, ARR, OBJ } type = NUL;
  bool b = false;
  double num = 0.0;
  bool integral = false;
  long long inum = 0;
  std::string s;
  std::vector<Json> arr;
  std::vector<std::pair<std::string, Json>> obj;
  const Json* get(const char* key) const {
    for (auto& kv : obj)
      if (kv.first == key) return &kv.second;
    return nullptr;
  }
};

struct Parser {
  const char* p;
  const char* end;
  std::string err;
  void ws() {
    while (p < end && (*p == ' ' || *p == '\t' || *p == '\n' || *p == '\r')) ++p;
  }
  bool fail(const char* m) {
    if (err.empty()) err = m;
    return false;
  }
  bool lit(const char* w) {
    const size_t n = std::strlen(w);
    if ((size_t)(end - p) < n || std::strncmp(p, w, n) != 0) return false;
    p += n;
    return true;
  }
  static void utf8(std::string& o, unsigned cp) {
    if (cp < 0x80) {
      o += (char)cp;
    } else if (cp < 0x800) {
      o += (char)(0xC0 | (cp >> 6));
      o += (char)(0x80 | (cp & 0x3F));
    } else if (cp < 0x10000) {
      o += (char)(0xE0 | (cp >> 12));
      o += (char)(0x80 | ((cp >> 6) & 0x3F));
      o += (char)(0x80 | (cp & 0x3F));
    } else {
      o += (char)(0xF0 | (cp >> 18));
      o += (char)(0x80 | ((cp >> 12) & 0x3F));
      o += (char)(0x80 | ((cp >> 6) & 0x3F));
      o += (char)(0x80 | (cp & 0x3F));
    }
  }
  bool hex4(unsigned& v) {
    if (end - p < 4) return false;
    v = 0;
    for (int i = 0; i < 4; ++i) {
      const char c = *p++;
      v <<= 4;
      if (c >= '0' && c <= '9') v |= (unsigned)(c - '0');
      else if (c >= 'a' && c <= 'f') v |= (unsigned)(c - 'a' + 10);
      else if (c >= 'A' && c <= 'F') v |= (unsigned)(c - 'A' + 10);
      else return false;
    }
    return true;
  }
  bool str(std::string& o) {
    if (p >= end || *p != '"') return fail("expected a string");
    ++p;
    while (p < end && *p != '"') {
      const unsigned char c = (unsigned char)*p;
      if (c < 0x20) return fail("control character in a string");
      if (c != '\\') {
        o += (char)c;
        ++p;
        continue;
      }
      if (++p >= end) return fail("unterminated escape");
      const char e = *p++;
      switch (e) {
        case '"': o += '"'; break;
        case '\\': o += '\\'; break;
        case '/': o += '/'; break;
        case 'b': o += '\b'; break;
        case 'f': o += '\f'; break;
        case 'n': o += '\n'; break;
        case 'r': o += '\r'; break;
        case 't': o += '\t'; break;
        case 'u': {
          unsigned cp;
          if (!hex4(cp)) return fail("bad \\u escape");
          if (cp >= 0xD800 && cp < 0xDC00) {  // a surrogate pair
            unsigned lo;
            if (!(lit("\\u") && hex4(lo) && lo >= 0xDC00 && lo < 0xE000)) return fail("bad surrogate pair");
            cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
          }
          utf8(o, cp);
          break;
        }
        default: return fail("bad escape");
      }
    }
    if (p >= end) return fail("unterminated string");
    ++p;
    return true;
  }
  bool value(Json& v, int depth) {
    if (depth > 64) return fail("nesting too deep");
    ws();
    if (p >= end) return fail("unexpected end");
    const char c = *p;
    if (c == '{') {
      ++p;
      v.type = Json::OBJ;
      ws();
      if (p < end && *p == '}') {
        ++p;
        return true;
      }
      for (;;) {
        ws();
        std::string k;
        if (!str(k)) return false;
        for (auto& kv : v.obj)
          if (kv.first == k) return fail("duplicate key");
        ws();
        if (p >= end || *p != ':') return fail("expected ':'");
        ++p;
        v.obj.emplace_back(k, Json{});
        if (!value(v.obj.back().second, depth + 1)) return false;
        ws();
        if (p < end && *p == ',') {
          ++p;
          continue;
        }
        if (p < end && *p == '}') {
          ++p;
          return true;
        }
        return fail("expected ',' or '}'");
      }
    }
    if (c == '[') {
      ++p;
      v.type = Json::ARR;
      ws();
      if (p < end && *p == ']') {
        ++p;
        return true;
      }
      for (;;) {
        v.arr.emplace_back();
        if (!value(v.arr.back(), depth + 1)) return false;
        ws();
        if (p < end && *p == ',') {
          ++p;
          continue;
        }
        if (p < end && *p == ']') {
          ++p;
          return true;
        }
        return fail("expected ',' or ']'");
      }
    }
    if (c == '"') {
      v.type = Json::STR;
      return str(v.s);
    }
    if (lit("true")) {
      v.type = Json::BOOL;
      v.b = true;
      return true;
    }
    if (lit("false")) {
      v.type = Json::BOOL;
      return true;
    }
    if (lit("null")) return true;
    // number
    const char* q = p;
    if (q < end && *q == '-') ++q;
    bool frac = false;
    while (q < end && ((*q >= '0' && *q <= '9') || *q == '.' || *q == 'e' || *q == 'E' || *q == '+' || *q == '-')) {
      if (*q == '.' || *q == 'e' || *q == 'E') frac = true;
      ++q;
    }
    if (q == p) return fail("unexpected character");
    const std::string t(p, q);
    char* e = nullptr;
    v.num = std::strtod(t.c_str(), &e);
    if (!e || *e) return fail("bad number");
    v.type = Json::NUM;
    if (!frac) {
      v.integral = true;
      v.inum = std::strtoll(t.c_str(), nullptr, 10);
    }
    p = q;
    return true;
  }
};

bool parse_json(const char* text, size_t len, Json& out, std::string& err) {
  Parser ps{text, text + len, {}};
  if (!ps.value(out, 0)) {
    err = ps.err;
    return false;
  }
  ps.ws();
  if (ps.p != ps.end) {
    err = "trailing characters after the JSON value";
    return false;
  }
  return true;
}

int msgf(char* msg, size_t n, int code, const char* fmt, ...) {
  if (msg && n) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, n, fmt, ap);
    va_end(ap);
  }
  return code;
}

// ---- numbers -------------------------------------------------------------------------------
float widen_f16(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = std::ldexp((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(1.0f + (float)m / 1024.0f, e - 15);
  return s ? -v : v;
}
float widen_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
uint16_t round_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---- the safetensors file ---------------------------------------------------------------------

constexpr uint64_t kMaxHeader = 1ull << 24;  // 16 MiB of JSON: far above a 28-layer index (~50 KB)

enum StType { ST_F32 = 0, ST_F16 = 1, ST_BF16 = 2, ST_U8 = 3 };
int st_size(int t) { return t == ST_F32 ? 4 : (t == ST_U8 ? 1 : 2); }

struct StTensor {
  std::string name;
  int type = ST_F32;
  std::vector<int64_t> shape;
  uint64_t begin = 0, end = 0;  // within the payload
};

struct StFile {
  const uint8_t* payload = nullptr;
  uint64_t payload_bytes = 0;
  std::map<std::string, StTensor> t;
  bool int4 = false;  // metadata quant = "int4-g32-sym"
  const StTensor* find(const std::string& n) const {
    auto it = t.find(n);
    return it == t.end() ? nullptr : &it->second;
  }
};

bool read_u64_le(const uint8_t* p, uint64_t& v) {
  v = 0;
  for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
  return true;
}

// F1 .. F7 on the mapped file; `why` says which rule failed.
bool parse_safetensors(const uint8_t* f, uint64_t size, StFile& out, std::string& why) {
  char b[256];
  if (size < 8) {  // F1
    why = "file of " + std::to_string(size) + " bytes has no room for the 8-byte header size";
    return false;
  }
  uint64_t n;
  read_u64_le(f, n);
  if (n < 2 || n > kMaxHeader || n > size - 8) {  // F2
    snprintf(b, sizeof b, "header size %llu is outside [2, %llu] or runs past the %llu-byte file",
             (unsigned long long)n, (unsigned long long)kMaxHeader, (unsigned long long)size);
    why = b;
    return false;
  }
  Json h;
  std::string err;
  if (!parse_json((const char*)f + 8, (size_t)n, h, err)) {  // F3 (the reader refuses repeated keys)
    why = "header JSON: " + err;
    return false;
  }
  if (h.type != Json::OBJ) {
    why = "header JSON is not an object";
    return false;
  }
  out.payload = f + 8 + n;
  out.payload_bytes = size - 8 - n;
  for (auto& kv : h.obj) {
    const std::string& name = kv.first;
    const Json& e = kv.second;
    if (name == "__metadata__") {  // F4
      if (e.type != Json::OBJ) {
        why = "__metadata__ is not an object";
        return false;
      }
      for (auto& m : e.obj) {
        if (m.second.type != Json::STR) {
          why = "__metadata__ entry " + m.first + " is not a string";
          return false;
        }
        if (m.first == "quant") {
          if (m.second.s != "int4-g32-sym") {
            why = "quant format " + m.second.s + " is not supported (only int4-g32-sym)";
            return false;
          }
          out.int4 = true;
        }
      }
      continue;
    }
    const Json* dt = e.type == Json::OBJ ? e.get("dtype") : nullptr;  // F5
    const Json* sh = e.type == Json::OBJ ? e.get("shape") : nullptr;
    const Json* of = e.type == Json::OBJ ? e.get("data_offsets") : nullptr;
    if (!dt || dt->type != Json::STR || !sh || sh->type != Json::ARR || !of || of->type != Json::ARR ||
        of->arr.size() != 2) {
      why = name + ": an entry needs a dtype string, a shape array and two data_offsets";
      return false;
    }
    StTensor t;
    t.name = name;
    static const std::pair<const char*, int> kTypes[] = {{"F32", ST_F32}, {"F16", ST_F16}, {"BF16", ST_BF16}, {"U8", ST_U8}};
    bool known = false;
    for (auto& ty : kTypes)
      if (dt->s == ty.first) {
        t.type = ty.second;
        known = true;
      }
    if (!known) {
      why = name + ": element type " + dt->s + " is not supported";
      return false;
    }
    uint64_t elems = 1;
    for (auto& d : sh->arr) {
      if (d.type != Json::NUM || !d.integral || d.inum < 0 || d.inum > (1ll << 40)) {
        why = name + ": shape entries must be non-negative integers";
        return false;
      }
      t.shape.push_back(d.inum);
      elems *= (uint64_t)d.inum;
      if (elems > (1ull << 40)) {
        why = name + ": shape too large";
        return false;
      }
    }
    for (auto& o : of->arr)
      if (o.type != Json::NUM || !o.integral || o.inum < 0) {
        why = name + ": data_offsets must be non-negative integers";
        return false;
      }
    t.begin = (uint64_t)of->arr[0].inum;
    t.end = (uint64_t)of->arr[1].inum;
    if (t.begin > t.end) {
      why = name + ": data_offsets end before they begin";
      return false;
    }
    if (t.end - t.begin != elems * (uint64_t)st_size(t.type)) {  // F6
      snprintf(b, sizeof b, ": %llu bytes stored, %llu needed by its shape and type",
               (unsigned long long)(t.end - t.begin), (unsigned long long)(elems * st_size(t.type)));
      why = name + b;
      return false;
    }
    out.t.emplace(name, std::move(t));
  }
  // F7: inside the payload, disjoint, and adding up to it
  std::vector<const StTensor*> byb;
  uint64_t total = 0;
  for (auto& kv : out.t) {
    if (kv.second.end > out.payload_bytes) {
      why = kv.first + ": data range runs past the end of the payload";
      return false;
    }
    total += kv.second.end - kv.second.begin;
    byb.push_back(&kv.second);
  }
  std::sort(byb.begin(), byb.end(), [](const StTensor* x, const StTensor* y) {
    return x->begin != y->begin ? x->begin < y->begin : x->end < y->end;
  });
  for (size_t i = 1; i < byb.size(); ++i)
    if (byb[i]->begin < byb[i - 1]->end) {
      why = "tensors " + byb[i - 1]->name + " and " + byb[i]->name + " share bytes";
      return false;
    }
  if (total != out.payload_bytes) {
    snprintf(b, sizeof b, "%llu payload bytes belong to no tensor", (unsigned long long)(out.payload_bytes - total));
    why = b;
    return false;
  }
  return true;
}

// element i of a float tensor, widened to float32
float st_float(const StFile& f, const StTensor& t, size_t i) {
  const uint8_t* d = f.payload + t.begin;
  if (t.type == ST_F32) {
    float x;
    std::memcpy(&x, d + 4 * i, 4);
    return x;
  }
  uint16_t x;
  std::memcpy(&x, d + 2 * i, 2);
  return t.type == ST_F16 ? widen_f16(x) : widen_bf16(x);
}

// ---- symmetric int4-g32 ("Candle model runner" 2.5), host side --------------------------------
// s = f16(max |w| / 7) with the quotient in float32 and round-to-nearest-even to f16; q =
// clamp(rint(w / s), -8, 7) with the float32 quotient and half-to-even rint; a group of zeros
// stores s = 0, q = 0. Two values per byte, column 2b in the low nibble, two's complement.
void quantize_int4_row(const float* w, int64_t cols, uint8_t* q, uint16_t* scale) {
  for (int64_t g = 0; g < cols / 32; ++g) {
    const float* x = w + g * 32;
    float mx = 0.f;
    for (int i = 0; i < 32; ++i) mx = std::max(mx, std::fabs(x[i]));
    const _Float16 sh = (_Float16)(mx / 7.0f);
    const float sf = (float)sh;
    std::memcpy(&scale[g], &sh, 2);
    for (int i = 0; i < 32; i += 2) {
      int v[2];
      for (int k = 0; k < 2; ++k) {
        const float r = sf > 0.f ? std::nearbyint(x[i + k] / sf) : 0.f;
        v[k] = (int)std::min(7.f, std::max(-8.f, r));
      }
      q[(g * 32 + i) / 2] = (uint8_t)((v[0] & 15) | ((v[1] & 15) << 4));
    }
  }
}

float int4_value(const uint8_t* q, const uint16_t* scale, int64_t cols, int64_t r, int64_t c) {
  const uint8_t byte = q[(r * cols + c) / 2];
  int v = (c & 1) ? byte >> 4 : byte & 15;
  if (v >= 8) v -= 16;
  _Float16 s;
  std::memcpy(&s, &scale[r * (cols / 32) + c / 32], 2);
  return (float)v * (float)s;  // exact: at most 15 significant bits
}

// ---- the checkpoint's names ------------------------------------------------------------------

// base name (without .weight / .qweight) of blob entry `idx` (entry layout of dec_weight_entry)
std::string hf_base(const dec_weight_info& e) {
  static const std::pair<const char*, const char*> kLayer[] = {
      {"attn_norm", "input_layernorm"}, {"wq", "self_attn.q_proj"},   {"wk", "self_attn.k_proj"},
      {"wv", "self_attn.v_proj"},       {"q_norm", "self_attn.q_norm"}, {"k_norm", "self_attn.k_norm"},
      {"wo", "self_attn.o_proj"},       {"ffn_norm", "post_attention_layernorm"},
      {"w_gate", "mlp.gate_proj"},      {"w_up", "mlp.up_proj"},       {"w_down", "mlp.down_proj"}};
  if (e.layer < 0) return std::strcmp(e.name, "embed") == 0 ? "model.embed_tokens" : "model.norm";
  for (auto& m : kLayer)
    if (std::strcmp(e.name, m.first) == 0) return "model.layers." + std::to_string(e.layer) + "." + m.second;
  return "";
}

bool same_shape(const StTensor& t, std::initializer_list<int64_t> want) {
  return t.shape.size() == want.size() && std::equal(want.begin(), want.end(), t.shape.begin());
}

std::string shape_str(const StTensor& t) {
  std::string s = "[";
  for (size_t i = 0; i < t.shape.size(); ++i) s += (i ? ", " : "") + std::to_string(t.shape[i]);
  return s + "]";
}

// A matrix source: a float tensor, or int4 values and scales.
struct MatSrc {
  const StTensor* w = nullptr;
  const StTensor* q = nullptr;
  const StTensor* s = nullptr;
  float at(const StFile& f, int64_t cols, int64_t r, int64_t c) const {
    if (w) return st_float(f, *w, (size_t)(r * cols + c));
    return int4_value(f.payload + q->begin, (const uint16_t*)(f.payload + s->begin), cols, r, c);
  }
};

// F8 for one matrix of shape [rows][cols] under base name b
bool find_matrix(const StFile& f, const std::string& b, int64_t rows, int64_t cols, MatSrc& m, std::string& why,
                 std::vector<std::string>& used) {
  if (f.int4) {
    m.q = f.find(b + ".qweight");
    m.s = f.find(b + ".scales");
    if (!m.q || !m.s) {
      why = "int4 file lacks " + b + ".qweight or " + b + ".scales";
      return false;
    }
    if (m.q->type != ST_U8 || !same_shape(*m.q, {rows, cols / 2})) {
      why = b + ".qweight must be U8 [" + std::to_string(rows) + ", " + std::to_string(cols / 2) + "], not " +
            shape_str(*m.q);
      return false;
    }
    if (m.s->type != ST_F16 || !same_shape(*m.s, {rows, cols / 32})) {
      why = b + ".scales must be F16 [" + std::to_string(rows) + ", " + std::to_string(cols / 32) + "], not " +
            shape_str(*m.s);
      return false;
    }
    used.push_back(b + ".qweight");
    used.push_back(b + ".scales");
    return true;
  }
  m.w = f.find(b + ".weight");
  if (!m.w) {
    why = "checkpoint lacks " + b + ".weight";
    return false;
  }
  if (m.w->type == ST_U8 || !same_shape(*m.w, {rows, cols})) {
    why = b + ".weight must be a float [" + std::to_string(rows) + ", " + std::to_string(cols) + "], not " +
          shape_str(*m.w);
    return false;
  }
  used.push_back(b + ".weight");
  return true;
}

// ---- config.json: the Qwen3 settings ("A real model in our own decoder"; refused at load:
// "Candle model runner" 2.3) -------------------------------------------------------------------
enum Want { W_STR, W_TRUE, W_FALSE, W_ZERO, W_NULL_OR_ABSENT };
struct Setting {
  const char* key;
  Want want;
  const char* str;  // for W_STR
};
// the architecture first, then what the forward pass leaves out, then the tie
const Setting kSettings[] = {
    {"model_type", W_STR, "qwen3"},          {"hidden_act", W_STR, "silu"},
    {"attention_bias", W_FALSE, nullptr},    {"attention_dropout", W_ZERO, nullptr},
    {"use_sliding_window", W_FALSE, nullptr}, {"rope_scaling", W_NULL_OR_ABSENT, nullptr},
    {"tie_word_embeddings", W_TRUE, nullptr},
};

bool setting_holds(const Json& j, const Setting& s) {
  const Json* x = j.get(s.key);
  switch (s.want) {
    case W_STR: return x && x->type == Json::STR && x->s == s.str;
    case W_TRUE: return x && x->type == Json::BOOL && x->b;
    case W_FALSE: return x && x->type == Json::BOOL && !x->b;
    case W_ZERO: return x && x->type == Json::NUM && x->num == 0.0;
    case W_NULL_OR_ABSENT: return !x || x->type == Json::NUL;
  }
  return false;
}

const char* setting_need(const Setting& s) {
  switch (s.want) {
    case W_STR: return s.str;
    case W_TRUE: return "true";
    case W_FALSE: return "false";
    case W_ZERO: return "0";
    case W_NULL_OR_ABSENT: return "null or absent";
  }
  return "";
}

}  // namespace

extern "C" {

int dec_config_from_json(const char* json, size_t len, dec_config* cfg, char* msg, size_t msg_len) {
  if (!json || !cfg) return msgf(msg, msg_len, DEC_E_ARG, "NULL argument");
  Json j;
  std::string err;
  if (!parse_json(json, len, j, err)) return msgf(msg, msg_len, DEC_E_ARG, "config.json does not parse: %s", err.c_str());
  if (j.type != Json::OBJ) return msgf(msg, msg_len, DEC_E_ARG, "config.json holds no object");
  for (const Setting& s : kSettings)
    if (!setting_holds(j, s))
      return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "config.json: %s must be %s for this decoder", s.key, setting_need(s));
  // shape fields, in the order of dec_config
  struct Field {
    const char* key;
    int32_t* dst;
  } fields[] = {{"num_hidden_layers", &cfg->n_layers},     {"hidden_size", &cfg->d_model},
                {"num_attention_heads", &cfg->n_heads},    {"num_key_value_heads", &cfg->n_kv_heads},
                {"head_dim", &cfg->head_dim},              {"intermediate_size", &cfg->ff_hidden},
                {"vocab_size", &cfg->vocab},               {"max_position_embeddings", &cfg->max_context}};
  int32_t vals[8];
  for (int i = 0; i < 8; ++i) {
    const Json* x = j.get(fields[i].key);
    if (!x || x->type != Json::NUM || !x->integral || x->inum < 1 || x->inum > 0x7fffffff)
      return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "config.json: %s needs a positive integer", fields[i].key);
    vals[i] = (int32_t)x->inum;
  }
  const Json* eps = j.get("rms_norm_eps");
  if (!eps || eps->type != Json::NUM || !(eps->num > 0.0) || !(eps->num < 1.0))
    return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "config.json: rms_norm_eps needs a number in (0, 1)");
  const Json* theta = j.get("rope_theta");
  if (!theta || theta->type != Json::NUM || !(theta->num > 1.0) || !std::isfinite(theta->num))
    return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "config.json: rope_theta needs a finite number above 1");
  for (int i = 0; i < 8; ++i) *fields[i].dst = vals[i];
  cfg->rms_eps = (float)eps->num;
  cfg->rope_base = theta->num;
  cfg->rope_split = cfg->qk_norm = cfg->tie_embeddings = 1;
  return msgf(msg, msg_len, DEC_OK, "");
}

int dec_load_safetensors(const char* path, const dec_config* cfg, void* blob, size_t blob_bytes, char* msg,
                         size_t msg_len) {
  if (!path || !cfg || !blob) return msgf(msg, msg_len, DEC_E_ARG, "NULL argument");
  if (dec_check_config(cfg) != DEC_OK) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "the configuration is refused");
  const int wd = cfg->weight_dtype;
  if (wd != DEC_F32 && wd != DEC_BF16 && wd != DEC_INT4_SYM_G32)
    return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "checkpoints load into float32, bf16 or symmetric int4-g32 blobs");
  if (blob_bytes < dec_weight_bytes(cfg)) return msgf(msg, msg_len, DEC_E_CAPACITY, "blob smaller than dec_weight_bytes");
  const int fd = open(path, O_RDONLY);
  if (fd < 0) return msgf(msg, msg_len, DEC_E_ARG, "cannot open %s", path);
  struct stat st;
  if (fstat(fd, &st) != 0 || st.st_size < 0) {
    close(fd);
    return msgf(msg, msg_len, DEC_E_ARG, "cannot stat %s", path);
  }
  const uint64_t fsz = (uint64_t)st.st_size;
  // (an empty file cannot be mapped; it fails F1)
  void* map = fsz ? mmap(nullptr, fsz, PROT_READ, MAP_PRIVATE, fd, 0) : nullptr;
  close(fd);
  if (fsz && map == MAP_FAILED) return msgf(msg, msg_len, DEC_E_ARG, "cannot map %s", path);
  auto finish = [&](int code, const std::string& why) {
    if (map) munmap(map, fsz);
    return msgf(msg, msg_len, code, "%s", why.c_str());
  };
  StFile f;
  std::string why;
  if (!parse_safetensors((const uint8_t*)map, fsz, f, why)) return finish(DEC_E_ARG, "model.safetensors: " + why);

  // F8: every blob entry from its tensor(s)
  const int n_entries = dec_weight_count(cfg);
  std::vector<dec_weight_info> ents(n_entries);
  std::vector<MatSrc> srcs(n_entries);
  std::vector<std::string> used;
  for (int i = 0; i < n_entries; ++i) {
    dec_weight_entry(cfg, i, &ents[i]);
    const dec_weight_info& e = ents[i];
    const std::string b = hf_base(e);
    if (e.rows == 1 && e.dtype == DEC_F32) {  // a gain vector
      const StTensor* t = f.find(b + ".weight");
      if (!t) return finish(DEC_E_ARG, "checkpoint lacks " + b + ".weight");
      if (t->type == ST_U8 || !same_shape(*t, {e.cols}))
        return finish(DEC_E_ARG, b + ".weight must be a float [" + std::to_string(e.cols) + "], not " + shape_str(*t));
      srcs[i].w = t;
      used.push_back(b + ".weight");
    } else if (!find_matrix(f, b, e.rows, e.cols, srcs[i], why, used)) {
      return finish(DEC_E_ARG, why);
    }
  }
  // F9: the tied matrix may be stored again, as lm_head; it must hold the embedding's values
  MatSrc lm;
  const bool has_lm = f.find("lm_head.weight") || f.find("lm_head.qweight") || f.find("lm_head.scales");
  if (has_lm && !find_matrix(f, "lm_head", ents[0].rows, ents[0].cols, lm, why, used)) return finish(DEC_E_ARG, why);
  std::sort(used.begin(), used.end());
  for (auto& kv : f.t)
    if (!std::binary_search(used.begin(), used.end(), kv.first))
      return finish(DEC_E_ARG, kv.first + " is not a tensor of this Qwen3 decoder");
  if (has_lm) {
    const int64_t R = ents[0].rows, C = ents[0].cols;
    for (int64_t r = 0; r < R; ++r)
      for (int64_t c = 0; c < C; ++c) {
        const float x = srcs[0].at(f, C, r, c), y = lm.at(f, C, r, c);
        if (!(x == y || (std::isnan(x) && std::isnan(y))))
          return finish(DEC_E_ARG, "lm_head differs from the tied embedding at [" + std::to_string(r) + ", " +
                                       std::to_string(c) + "]");
      }
  }

  // fill the blob: gains as float32; matrices in the blob's format
  uint8_t* out = (uint8_t*)blob;
  std::vector<float> row;
  for (int i = 0; i < n_entries; ++i) {
    const dec_weight_info& e = ents[i];
    const MatSrc& m = srcs[i];
    const int64_t R = e.rows, C = e.cols;
    if (e.dtype == DEC_F32) {  // gains (any blob) and float32 matrices
      float* o = (float*)(out + e.offset);
      for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) o[r * C + c] = m.at(f, C, r, c);
    } else if (e.dtype == DEC_BF16) {
      uint16_t* o = (uint16_t*)(out + e.offset);
      if (m.w && m.w->type == ST_BF16) {
        std::memcpy(o, f.payload + m.w->begin, (size_t)(R * C) * 2);  // as stored
      } else {
        for (int64_t r = 0; r < R; ++r)
          for (int64_t c = 0; c < C; ++c) o[r * C + c] = round_bf16(m.at(f, C, r, c));
      }
    } else {  // DEC_INT4_SYM_G32: copied from an int4 file, or quantised at load
      uint8_t* q = out + e.offset;
      uint16_t* sc = (uint16_t*)(out + e.scale_offset);
      if (m.q) {
        std::memcpy(q, f.payload + m.q->begin, (size_t)(R * C / 2));
        std::memcpy(sc, f.payload + m.s->begin, (size_t)(R * (C / 32)) * 2);
      } else {
        row.resize((size_t)C);
        for (int64_t r = 0; r < R; ++r) {
          for (int64_t c = 0; c < C; ++c) row[c] = m.at(f, C, r, c);
          quantize_int4_row(row.data(), C, q + r * (C / 2), sc + r * (C / 32));
        }
      }
    }
  }
  return finish(DEC_OK, "");
}

}  // extern "C"
