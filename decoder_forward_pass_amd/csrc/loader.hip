// Checkpoint loading (host only): config.json of a Qwen3 model into a dec_config, and a
// model.safetensors file into the library's weights blob.
//
// config.json: the settings "A real model in our own decoder" whitelists (qwen_config: model type
// qwen3, silu, no attention bias or dropout, no RoPE scaling, no sliding window, tied
// embeddings, RMSNorm eps 1e-6) must hold, else the model is refused; the shape fields must be
// positive integers ("Candle model runner" 2.3: what the engine cannot run is refused at load).
//
// model.safetensors ("A real model in our own decoder", section "A safetensors file is a JSON
// header and raw bytes"; "Candle model runner" 2.3): a little-endian u64 header length N, N
// bytes of JSON, then the data buffer. Refused: N outside [2, min(1e8, file size - 8)], a header
// that is not one object, duplicate keys, metadata that is not strings, an unknown dtype, a byte
// count that does not match the shape, ranges (counted from the start of the data buffer) that
// overlap, leave a gap or do not end at the end of the file. Tensors arrive as F32, F16 or BF16
// and are widened to float32 ("Candle model runner" 2.3 widening equations), then stored in the
// blob's dtype (bf16: rounded to nearest even). The tied output matrix may be stored a second
// time as lm_head.weight; it must then equal the embedding ("A real model in our own decoder",
// section "Two things the real file taught us").
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

struct Tensor {
  int dtype;  // 0 F32, 1 F16, 2 BF16
  std::vector<int64_t> shape;
  size_t start, end;  // from the start of the data buffer
};

int dtype_size(int d) { return d == 0 ? 4 : 2; }

}  // namespace

extern "C" {

int dec_config_from_json(const char* json, size_t len, dec_config* cfg, char* msg, size_t msg_len) {
  if (!json || !cfg) return msgf(msg, msg_len, DEC_E_ARG, "NULL argument");
  Json j;
  std::string err;
  if (!parse_json(json, len, j, err)) return msgf(msg, msg_len, DEC_E_ARG, "config.json: %s", err.c_str());
  if (j.type != Json::OBJ) return msgf(msg, msg_len, DEC_E_ARG, "config.json is not an object");
  auto is_str = [&](const char* k, const char* v) {
    const Json* x = j.get(k);
    return x && x->type == Json::STR && x->s == v;
  };
  auto is_bool = [&](const char* k, bool v) {
    const Json* x = j.get(k);
    return x && x->type == Json::BOOL && x->b == v;
  };
  auto is_num = [&](const char* k, double v) {
    const Json* x = j.get(k);
    return x && x->type == Json::NUM && x->num == v;
  };
  auto is_null = [&](const char* k) {
    const Json* x = j.get(k);
    return !x || x->type == Json::NUL;
  };
  if (!is_str("model_type", "qwen3")) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "unsupported setting: model_type");
  if (!is_str("hidden_act", "silu")) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "unsupported setting: hidden_act");
  if (!is_bool("attention_bias", false)) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "unsupported setting: attention_bias");
  if (!is_num("attention_dropout", 0.0)) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "unsupported setting: attention_dropout");
  if (!is_null("rope_scaling")) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "unsupported setting: rope_scaling");
  if (!is_bool("use_sliding_window", false)) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "unsupported setting: use_sliding_window");
  if (!is_bool("tie_word_embeddings", true)) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "unsupported setting: tie_word_embeddings");
  if (!is_num("rms_norm_eps", 1e-6)) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "unsupported setting: rms_norm_eps");
  int32_t v[8];
  const char* names[8] = {"vocab_size", "max_position_embeddings", "hidden_size", "num_attention_heads",
                          "num_hidden_layers", "num_key_value_heads", "head_dim", "intermediate_size"};
  for (int i = 0; i < 8; ++i) {
    const Json* x = j.get(names[i]);
    if (!x || x->type != Json::NUM || !x->integral || x->inum < 1 || x->inum > 0x7fffffff)
      return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "%s must be a positive integer", names[i]);
    v[i] = (int32_t)x->inum;
  }
  const Json* rt = j.get("rope_theta");
  if (!rt || rt->type != Json::NUM || !(rt->num > 1.0)) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "rope_theta must be a number > 1");
  cfg->vocab = v[0];
  cfg->max_context = v[1];
  cfg->d_model = v[2];
  cfg->n_heads = v[3];
  cfg->n_layers = v[4];
  cfg->n_kv_heads = v[5];
  cfg->head_dim = v[6];
  cfg->ff_hidden = v[7];
  cfg->rms_eps = 1e-6f;
  cfg->rope_base = rt->num;
  cfg->rope_split = cfg->qk_norm = cfg->tie_embeddings = 1;
  return msgf(msg, msg_len, DEC_OK, "");
}

int dec_load_safetensors(const char* path, const dec_config* cfg, void* blob, size_t blob_bytes, char* msg,
                         size_t msg_len) {
  if (!path || !cfg || !blob) return msgf(msg, msg_len, DEC_E_ARG, "NULL argument");
  if (dec_check_config(cfg) != DEC_OK) return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "the configuration is refused");
  if (cfg->weight_dtype != DEC_F32 && cfg->weight_dtype != DEC_BF16)
    return msgf(msg, msg_len, DEC_E_UNSUPPORTED, "loading fills float32 or bf16 blobs");
  if (blob_bytes < dec_weight_bytes(cfg)) return msgf(msg, msg_len, DEC_E_CAPACITY, "blob smaller than dec_weight_bytes");
  const int fd = open(path, O_RDONLY);
  if (fd < 0) return msgf(msg, msg_len, DEC_E_ARG, "cannot open %s", path);
  struct stat stt;
  if (fstat(fd, &stt) != 0) {
    close(fd);
    return msgf(msg, msg_len, DEC_E_ARG, "cannot stat %s", path);
  }
  const size_t fsz = (size_t)stt.st_size;
  if (fsz < 8) {
    close(fd);
    return msgf(msg, msg_len, DEC_E_ARG, "truncated safetensors header length");
  }
  void* map = mmap(nullptr, fsz, PROT_READ, MAP_PRIVATE, fd, 0);
  close(fd);
  if (map == MAP_FAILED) return msgf(msg, msg_len, DEC_E_ARG, "cannot map %s", path);
  const uint8_t* f = (const uint8_t*)map;
  auto done = [&](int code, const char* fmt, const char* a = "") {
    munmap(map, fsz);
    return msgf(msg, msg_len, code, fmt, a);
  };
  uint64_t n = 0;
  for (int i = 0; i < 8; ++i) n |= (uint64_t)f[i] << (8 * i);
  if (n < 2 || n > 100000000ull || n > fsz - 8) return done(DEC_E_ARG, "invalid safetensors header length");
  Json h;
  std::string err;
  if (!parse_json((const char*)f + 8, (size_t)n, h, err)) return done(DEC_E_ARG, "safetensors header: %s", err.c_str());
  if (h.type != Json::OBJ) return done(DEC_E_ARG, "safetensors header must be an object");
  std::map<std::string, Tensor> ts;
  for (auto& kv : h.obj) {
    if (kv.first == "__metadata__") {
      if (kv.second.type != Json::OBJ) return done(DEC_E_ARG, "invalid safetensors metadata");
      for (auto& m : kv.second.obj)
        if (m.second.type != Json::STR) return done(DEC_E_ARG, "invalid safetensors metadata");
      continue;
    }
    const Json& e = kv.second;
    const Json* dt = e.type == Json::OBJ ? e.get("dtype") : nullptr;
    const Json* sh = e.type == Json::OBJ ? e.get("shape") : nullptr;
    const Json* of = e.type == Json::OBJ ? e.get("data_offsets") : nullptr;
    if (!dt || dt->type != Json::STR || !sh || sh->type != Json::ARR || !of || of->type != Json::ARR || of->arr.size() != 2)
      return done(DEC_E_ARG, "tensor %s: needs dtype, shape and data_offsets", kv.first.c_str());
    Tensor t;
    if (dt->s == "F32") t.dtype = 0;
    else if (dt->s == "F16") t.dtype = 1;
    else if (dt->s == "BF16") t.dtype = 2;
    else return done(DEC_E_ARG, "tensor %s: unknown or unsupported dtype", kv.first.c_str());
    uint64_t count = 1;
    for (auto& d : sh->arr) {
      if (d.type != Json::NUM || !d.integral || d.inum < 0) return done(DEC_E_ARG, "tensor %s: bad shape", kv.first.c_str());
      t.shape.push_back(d.inum);
      count *= (uint64_t)d.inum;
    }
    for (auto& o : of->arr)
      if (o.type != Json::NUM || !o.integral || o.inum < 0) return done(DEC_E_ARG, "tensor %s: bad data_offsets", kv.first.c_str());
    t.start = (size_t)of->arr[0].inum;
    t.end = (size_t)of->arr[1].inum;
    if (t.end < t.start || t.end - t.start != count * dtype_size(t.dtype))
      return done(DEC_E_ARG, "tensor %s: byte count does not match its shape", kv.first.c_str());
    ts[kv.first] = t;
  }
  // the ranges tile the data buffer: sorted by (start, end), each starts where the last ended
  std::vector<std::pair<size_t, size_t>> rs;
  for (auto& kv : ts) rs.emplace_back(kv.second.start, kv.second.end);
  std::sort(rs.begin(), rs.end());
  size_t cursor = 0;
  for (auto& r : rs) {
    if (r.first != cursor) return done(DEC_E_ARG, "tensor offsets overlap or leave a gap");
    cursor = r.second;
  }
  const size_t data0 = 8 + (size_t)n;
  if (cursor != fsz - data0) return done(DEC_E_ARG, "tensor offsets do not cover the complete payload");

  // names of the checkpoint and where they go in the blob
  const int L = cfg->n_layers;
  const int count_entries = dec_weight_count(cfg);
  std::map<std::string, int> want;  // checkpoint name -> blob entry
  want["model.embed_tokens.weight"] = 0;
  const char* per[11] = {"input_layernorm.weight",  "self_attn.q_proj.weight", "self_attn.k_proj.weight",
                         "self_attn.v_proj.weight", "self_attn.q_norm.weight", "self_attn.k_norm.weight",
                         "self_attn.o_proj.weight", "post_attention_layernorm.weight", "mlp.gate_proj.weight",
                         "mlp.up_proj.weight",      "mlp.down_proj.weight"};
  for (int l = 0; l < L; ++l)
    for (int i = 0; i < 11; ++i) want["model.layers." + std::to_string(l) + "." + per[i]] = 1 + l * 11 + i;
  want["model.norm.weight"] = 1 + L * 11;
  if (count_entries != 2 + L * 11) return done(DEC_E_UNSUPPORTED, "unexpected blob layout");
  for (auto& kv : ts)
    if (!want.count(kv.first) && kv.first != "lm_head.weight")
      return done(DEC_E_ARG, "unexpected checkpoint tensor: %s", kv.first.c_str());
  for (auto& kv : want)
    if (!ts.count(kv.first)) return done(DEC_E_ARG, "missing checkpoint tensor: %s", kv.first.c_str());
  auto value = [&](const Tensor& t, size_t i) -> float {
    const uint8_t* d = f + data0 + t.start;
    if (t.dtype == 0) {
      float x;
      std::memcpy(&x, d + 4 * i, 4);
      return x;
    }
    uint16_t x;
    std::memcpy(&x, d + 2 * i, 2);
    return t.dtype == 1 ? widen_f16(x) : widen_bf16(x);
  };
  uint8_t* out = (uint8_t*)blob;
  for (auto& kv : want) {
    dec_weight_info e;
    dec_weight_entry(cfg, kv.second, &e);
    const Tensor& t = ts[kv.first];
    const bool vec = e.rows == 1 && e.dtype == DEC_F32 && std::strstr(e.name, "norm");
    const bool shape_ok = vec ? (t.shape.size() == 1 && t.shape[0] == e.cols)
                              : (t.shape.size() == 2 && t.shape[0] == e.rows && t.shape[1] == e.cols);
    if (!shape_ok) return done(DEC_E_ARG, "checkpoint tensor shape mismatch: %s", kv.first.c_str());
    const size_t cnt = (size_t)e.rows * e.cols;
    if (e.dtype == DEC_F32) {
      float* o = (float*)(out + e.offset);
      for (size_t i = 0; i < cnt; ++i) o[i] = value(t, i);
    } else {
      uint16_t* o = (uint16_t*)(out + e.offset);
      if (t.dtype == 2)
        std::memcpy(o, f + data0 + t.start, cnt * 2);  // bf16 as stored
      else
        for (size_t i = 0; i < cnt; ++i) o[i] = round_bf16(value(t, i));
    }
  }
  // a stored lm_head.weight must be the embedding again (as values)
  auto lm = ts.find("lm_head.weight");
  if (lm != ts.end()) {
    const Tensor& a = ts["model.embed_tokens.weight"];
    const Tensor& b = lm->second;
    if (b.shape != a.shape) return done(DEC_E_ARG, "checkpoint tied weights differ");
    const size_t cnt = (size_t)a.shape[0] * a.shape[1];
    for (size_t i = 0; i < cnt; ++i) {
      const float x = value(a, i), y = value(b, i);
      if (!(x == y || (std::isnan(x) && std::isnan(y)))) return done(DEC_E_ARG, "checkpoint tied weights differ");
    }
  }
  munmap(map, fsz);
  return msgf(msg, msg_len, DEC_OK, "");
}

}  // extern "C"
