// Host runtime of the C ABI in dec.h: configuration checks, blob / pool / workspace
// layout, validation of every call before anything is enqueued, the pinned metadata ring,
// the RoPE table, and the per-call launch sequence on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using namespace dec;

namespace {

thread_local std::string g_err;  // message of the last failure without a ctx

constexpr size_t kAlign = 256;
constexpr int kSlots = 4;  // pinned metadata staging slots
constexpr int kPerLayer = 11;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int fail(std::string* err, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (err) *err = buf;
  return code;
}

int check_config(const dec_config* c, std::string* err) {
  if (!c) return fail(err, DEC_E_ARG, "config is NULL");
  if (c->rope_split != 1) return fail(err, DEC_E_UNSUPPORTED, "rope_split must be 1 (pairs j, j + head_dim/2)");
  if (c->qk_norm != 1) return fail(err, DEC_E_UNSUPPORTED, "qk_norm must be 1");
  if (c->tie_embeddings != 1) return fail(err, DEC_E_UNSUPPORTED, "tie_embeddings must be 1");
  if (c->n_layers < 1) return fail(err, DEC_E_UNSUPPORTED, "n_layers must be >= 1");
  if (c->d_model < 64 || c->d_model % 64) return fail(err, DEC_E_UNSUPPORTED, "d_model must be a positive multiple of 64");
  if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
    return fail(err, DEC_E_UNSUPPORTED, "n_heads must be a positive multiple of n_kv_heads");
  const int group = c->n_heads / c->n_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(err, DEC_E_UNSUPPORTED, "n_heads / n_kv_heads must be 1, 2, 4 or 8");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(err, DEC_E_UNSUPPORTED, "head_dim must be 32, 64 or 128");
  if ((c->n_heads * c->head_dim) % 64 || (c->n_kv_heads * c->head_dim) % 64)
    return fail(err, DEC_E_UNSUPPORTED, "n_heads*head_dim and n_kv_heads*head_dim must be multiples of 64");
  if (c->ff_hidden < 64 || c->ff_hidden % 64) return fail(err, DEC_E_UNSUPPORTED, "ff_hidden must be a positive multiple of 64");
  if (c->vocab < 1) return fail(err, DEC_E_UNSUPPORTED, "vocab must be >= 1");
  if (c->max_context < 1) return fail(err, DEC_E_UNSUPPORTED, "max_context must be >= 1");
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return fail(err, DEC_E_UNSUPPORTED, "rms_eps must be positive");
  if (!(c->rope_base > 1.0) || !std::isfinite(c->rope_base)) return fail(err, DEC_E_UNSUPPORTED, "rope_base must be > 1");
  if (c->weight_dtype != DEC_F32 && c->weight_dtype != DEC_BF16 && c->weight_dtype != DEC_UINT4_G32 &&
      c->weight_dtype != DEC_INT4_SYM_G32)
    return fail(err, DEC_E_UNSUPPORTED, "weight_dtype must be DEC_F32, DEC_BF16, DEC_UINT4_G32 or DEC_INT4_SYM_G32");
  if (c->kv_dtype != DEC_F32 && c->kv_dtype != DEC_F16) return fail(err, DEC_E_UNSUPPORTED, "kv_dtype must be DEC_F32 or DEC_F16");
  if (c->block_tokens != 16 && c->block_tokens != 32 && c->block_tokens != 64)
    return fail(err, DEC_E_UNSUPPORTED, "block_tokens must be 16, 32 or 64");
  if (c->n_blocks < 1) return fail(err, DEC_E_UNSUPPORTED, "n_blocks must be >= 1 (a pool without blocks is refused)");
  if (c->max_rows < 1 || c->max_seqs < 1 || c->max_seqs > c->max_rows)
    return fail(err, DEC_E_UNSUPPORTED, "need 1 <= max_seqs <= max_rows");
  // (the host orders decode attention work items by row * 4096 + segment, in 32 bits)
  if ((int64_t)c->max_context > (int64_t)kDecodeSegKeys * kDecodeMaxSegs)
    return fail(err, DEC_E_UNSUPPORTED, "max_context must be <= %d", kDecodeSegKeys * kDecodeMaxSegs);
  if (c->max_seqs > (1 << 19)) return fail(err, DEC_E_UNSUPPORTED, "max_seqs must be <= 524288");
  return DEC_OK;
}

// ---- weights blob layout -------------------------------------------------------------------

struct Blob {
  std::vector<dec_weight_info> e;
  size_t total = 0;
};

Blob blob_layout(const dec_config& c) {
  Blob b;
  size_t off = 0;
  auto gain = [&](const char* name, int layer, int64_t n) {
    dec_weight_info w{};
    snprintf(w.name, sizeof w.name, "%s", name);
    w.layer = layer;
    w.dtype = DEC_F32;
    w.rows = 1;
    w.cols = n;
    w.offset = off;
    w.bytes = (size_t)n * 4;
    off = align_up(off + w.bytes);
    b.e.push_back(w);
  };
  auto mat = [&](const char* name, int layer, int64_t rows, int64_t cols) {
    dec_weight_info w{};
    snprintf(w.name, sizeof w.name, "%s", name);
    w.layer = layer;
    w.dtype = c.weight_dtype;
    w.rows = rows;
    w.cols = cols;
    w.offset = off;
    if (c.weight_dtype == DEC_UINT4_G32) {
      w.bytes = (size_t)(rows * cols / 2);
      w.group_bytes = (size_t)(rows * (cols / 32) * 2);
      w.scale_offset = align_up(off + w.bytes);
      w.zp_offset = align_up(w.scale_offset + w.group_bytes);
      off = align_up(w.zp_offset + w.group_bytes);
    } else if (c.weight_dtype == DEC_INT4_SYM_G32) {
      w.bytes = (size_t)(rows * cols / 2);
      w.group_bytes = (size_t)(rows * (cols / 32) * 2);
      w.scale_offset = align_up(off + w.bytes);
      off = align_up(w.scale_offset + w.group_bytes);
    } else {
      w.bytes = (size_t)(rows * cols * (c.weight_dtype == DEC_F32 ? 4 : 2));
      off = align_up(off + w.bytes);
    }
    b.e.push_back(w);
  };
  const int64_t d = c.d_model, qw = (int64_t)c.n_heads * c.head_dim, kvw = (int64_t)c.n_kv_heads * c.head_dim;
  mat("embed", -1, c.vocab, d);
  for (int l = 0; l < c.n_layers; ++l) {
    gain("attn_norm", l, d);
    mat("wq", l, qw, d);
    mat("wk", l, kvw, d);
    mat("wv", l, kvw, d);
    gain("q_norm", l, c.head_dim);
    gain("k_norm", l, c.head_dim);
    mat("wo", l, d, qw);
    gain("ffn_norm", l, d);
    mat("w_gate", l, c.ff_hidden, d);
    mat("w_up", l, c.ff_hidden, d);
    mat("w_down", l, d, c.ff_hidden);
  }
  gain("final_norm", -1, d);
  b.total = off;
  return b;
}

size_t kv_bytes(const dec_config& c) {
  return (size_t)c.n_layers * 2 * (size_t)c.n_blocks * c.n_kv_heads * c.block_tokens * c.head_dim *
         (c.kv_dtype == DEC_F32 ? 4 : 2);
}

// ---- workspace layout ----------------------------------------------------------------------

struct Ws {
  size_t rope, meta, x, h, qkv, q, o, a, part, dpart, amax, ssq, xg, samp, counts, wide, fpart, total;
  size_t meta_ints;  // capacity of the metadata region in int32
  size_t wide_bytes;  // the widened-layer region (0: calls never widen)
  size_t fpart_floats;  // float32 weights: the K-part sums of split products (0: none)
  int chunk, nch_max, max_blocks_per_seq, max_tiles;
  int seg_keys, dslots;  // decode attention: keys per segment; state slots per (row, KV head)
  int act_bytes, kv_el;
  bool flash;  // prefill attention by the MFMA tile kernel
};

// Prefill calls of at least this many rows with 4-bit weights widen each layer's matrices to bf16
// first (the rows' products then fill the chip with the larger bf16 tiles)
constexpr int kWidenRows = 4096;

// `decode_rows` > 0: only the regions a decode step of that many sequences uses (no RoPE table,
// no prefill partials, no sampler regions), laid out for those rows: the static scratch of
// dec_decode_step_static
Ws ws_layout(const dec_config& c, int decode_rows = 0) {
  Ws w{};
  const bool dec_only = decode_rows > 0;
  const size_t R = dec_only ? (size_t)decode_rows : (size_t)c.max_rows, S = dec_only ? (size_t)decode_rows : (size_t)c.max_seqs;
  const size_t d = c.d_model, D = c.head_dim, H = c.n_heads;
  const size_t qw = H * D, qkvw = qw + 2 * (size_t)c.n_kv_heads * D, ff = c.ff_hidden;
  w.act_bytes = c.weight_dtype == DEC_F32 ? 4 : 2;
  w.kv_el = c.kv_dtype == DEC_F32 ? 4 : 2;
  w.max_blocks_per_seq = (c.max_context + c.block_tokens - 1) / c.block_tokens;
  w.max_tiles = (int)(R / 64 + S);
  w.chunk = attn_rows_chunk(c.head_dim, c.kv_dtype == DEC_F16, c.n_heads / c.n_kv_heads);
  w.nch_max = w.chunk ? (c.max_context + w.chunk - 1) / w.chunk : 0;
  w.seg_keys = std::max(kDecodeSegKeys, c.block_tokens);
  w.dslots = (c.max_context + w.seg_keys - 1) / w.seg_keys + 1;
  w.meta_ints = 3 * R + 3 * S + R + 2 * (size_t)w.max_tiles + S * (size_t)w.max_blocks_per_seq + 3 +
                4 * S * (size_t)(w.dslots - 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  w.rope = take(dec_only ? 0 : (size_t)c.max_context * (D / 2) * sizeof(float2));
  w.meta = take(w.meta_ints * 4);
  w.x = take(R * d * 4);
  w.h = take(R * d * w.act_bytes);
  w.qkv = take(std::max(R, S) * qkvw * 4);  // float32 Q|K|V product
  w.q = take(R * qw * w.kv_el);
  w.o = take(R * qw * w.act_bytes);
  w.a = take(R * ff * w.act_bytes);
  // split-key partials: only prefill calls that take the per-row kernel (float32 pool, or a
  // head shape the tile kernel does not take) use them; decode merges its chunks in-block
  w.flash = c.kv_dtype == DEC_F16 && attn_prefill_supported(c.head_dim, c.n_heads / c.n_kv_heads);
  const size_t prow = w.flash || dec_only ? 0 : R;
  w.part = take(prow * H * (size_t)w.nch_max * (D + 2) * 4);
  // decode rows split into segments: one state per (row, KV head, segment), plus the new key's
  w.dpart = take(S * H * (size_t)w.dslots * (D + 2) * 4);
  w.amax = take(argmax_scratch_bytes((int)R, (int)S));
  w.ssq = take(S * (d / 16) * 4);  // decode: sums of squares of the residual in 16-column partials
  w.xg = take(S * d * 2);          // decode: bf16(residual * the next norm's gain)
  w.samp = take(dec_only ? 0 : S * sizeof(SampleSeq));       // sampling: per-sequence parameters and history
  w.counts = take(dec_only ? 0 : S * (size_t)c.vocab * 4);   // sampling: per-sequence count table (kept zero)
  // 4-bit weights: one layer's matrices widened to bf16, for prefill calls of at least kWidenRows
  const bool wide = !dec_only && is_q4(c.weight_dtype) && c.max_rows >= kWidenRows;
  w.wide_bytes = wide ? (qkvw * d + d * qw + 2 * ff * d + d * ff) * 2 : 0;
  w.wide = take(w.wide_bytes);
  // float32 weights: a product whose grid of 64 x 64 tiles is under 256 splits K into its parts
  // over blocks (m tiles * n tiles < 256), f32_k_parts(epi) * matrices * M * N floats of sums; the
  // largest over the products for calls of up to R rows (none in the static decode scratch:
  // those products then take the unsplit kernel, with the same results)
  w.fpart_floats = 0;
  if (c.weight_dtype == DEC_F32 && !dec_only) {
    auto need = [&](int epi, size_t N, size_t nb) -> size_t {
      const size_t mt = 255 / ((N + 63) / 64);
      return f32_k_parts(epi) * nb * std::min(R, 64 * mt) * N;
    };
    w.fpart_floats = std::max({need(EPI_STORE, qkvw, 1), need(EPI_RESID, d, 1), need(EPI_SWIGLU, ff, 2),
                               need(EPI_STORE, (size_t)c.vocab, 1)});
  }
  w.fpart = take(w.fpart_floats * 4);
  w.total = off;
  return w;
}

struct LayerW {
  const float *attn_norm, *q_norm, *k_norm, *ffn_norm;
  WMat wq, wk, wv, wo, wg, wu, wd;
};

// Validation of one step; shared by dec_check_step, dec_prefill and dec_decode_step.
int check_step(const dec_config& c, int32_t S, const int32_t* start, const int32_t* n_new,
               const int32_t* tokens, const int32_t* tables, int32_t max_blocks, int32_t mode,
               std::string* err) {
  if (S <= 0) return fail(err, DEC_E_ARG, "n_seqs must be >= 1");
  if (S > c.max_seqs) return fail(err, DEC_E_CAPACITY, "n_seqs %d exceeds max_seqs %d", S, c.max_seqs);
  if (!start) return fail(err, DEC_E_ARG, "start/positions is NULL");
  if (!tables) return fail(err, DEC_E_ARG, "block_tables is NULL");
  if (max_blocks <= 0) return fail(err, DEC_E_ARG, "max_blocks must be >= 1");
  if (mode != DEC_LOGITS_ALL && mode != DEC_LOGITS_LAST && mode != DEC_LOGITS_NONE)
    return fail(err, DEC_E_ARG, "unknown logits mode %d", mode);
  int64_t N = 0;
  for (int s = 0; s < S; ++s) {
    const int64_t n = n_new ? n_new[s] : 1;
    if (n < 1) return fail(err, DEC_E_ARG, "sequence %d: n_new must be >= 1", s);
    if (start[s] < 0) return fail(err, DEC_E_POSITION, "sequence %d: start %d is negative", s, start[s]);
    if ((int64_t)start[s] + n > c.max_context)
      return fail(err, DEC_E_POSITION, "sequence %d: positions up to %lld pass max_context %d", s,
                  (long long)(start[s] + n - 1), c.max_context);
    N += n;
  }
  if (N > c.max_rows) return fail(err, DEC_E_CAPACITY, "%lld new tokens exceed max_rows %d", (long long)N, c.max_rows);
  if (tokens) {
    for (int64_t i = 0; i < N; ++i)
      if (tokens[i] < 0 || tokens[i] >= c.vocab)
        return fail(err, DEC_E_TOKEN, "token %lld: id %d outside [0, %d)", (long long)i, tokens[i], c.vocab);
  }
  // blocks: table long enough, ids in range, blocks receiving new positions not shared
  std::vector<std::pair<int32_t, int32_t>> written;
  for (int s = 0; s < S; ++s) {
    const int64_t n = n_new ? n_new[s] : 1;
    const int64_t need = (start[s] + n + c.block_tokens - 1) / c.block_tokens;
    if (need > max_blocks)
      return fail(err, DEC_E_BLOCK, "sequence %d: block table of %d entries, %lld needed", s, max_blocks, (long long)need);
    const int32_t* row = tables + (int64_t)s * max_blocks;
    for (int64_t j = 0; j < need; ++j)
      if (row[j] < 0 || row[j] >= c.n_blocks)
        return fail(err, DEC_E_BLOCK, "sequence %d: block id %d at table entry %lld outside [0, %d)", s, row[j],
                    (long long)j, c.n_blocks);
    for (int64_t j = start[s] / c.block_tokens; j < need; ++j) written.push_back({row[j], s});
  }
  std::sort(written.begin(), written.end());
  for (size_t i = 1; i < written.size(); ++i)
    if (written[i].first == written[i - 1].first && written[i].second != written[i - 1].second)
      return fail(err, DEC_E_BLOCK, "block %d receives new positions of sequences %d and %d", written[i].first,
                  written[i - 1].second, written[i].second);
  return DEC_OK;
}

}  // namespace

// Event pairs around launches of the timed kernel classes.
struct Timing {
  uint32_t mask = 0;
  std::vector<hipEvent_t> pool;                       // free events
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec[DEC_K_COUNT];
};

struct dec_ctx {
  Timing timing;
  dec_config cfg;
  Blob blob;
  Ws ws;
  const uint8_t* w;
  void* pool;
  uint8_t* wsp;
  std::vector<LayerW> layers;
  WMat embed;
  const float* final_norm;
  int32_t* staging[kSlots];
  hipEvent_t ev[kSlots];
  int slot;
  SampleSeq* samp_staging;  // pinned: the last dec_sample call's parameters
  hipEvent_t samp_ev;       // that upload's completion
  void* scratch;            // device address of this device's static scratch (dec_decode_step_static)
  std::string scratch_err;  // why it is unknown, when it is
  std::string err;
};

namespace {

// The static scratch of dec_decode_step_static: per-call device memory (metadata, activations,
// split attention states, greedy candidates) for callers that cannot allocate. One copy per
// device, held until the process ends; every call on a device shares it. Host code never passes
// the array's name to a kernel or a copy (there it is a host-side stand-in): it uses the device
// address hipGetSymbolAddress gives for the current device, kept per device.
constexpr size_t kStaticScratchBytes = DEC_STATIC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// The current device's static scratch address (looked up once per device), or nullptr with `why`.
void* static_scratch(std::string* why) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *why = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *why = "device index beyond the static scratch table";
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *why = std::string("hipGetSymbolAddress: ") + hipGetErrorString(e);
      return nullptr;
    }
    g_scratch_addr[dev] = p;
  }
  return g_scratch_addr[dev];
}

}  // namespace

namespace {

WMat wmat(const dec_ctx* c, int idx) {
  const dec_weight_info& e = c->blob.e[idx];
  WMat m;
  m.w = c->w + e.offset;
  m.scale = e.dtype == DEC_UINT4_G32 || e.dtype == DEC_INT4_SYM_G32 ? (const uint16_t*)(c->w + e.scale_offset) : nullptr;
  m.zp = e.dtype == DEC_UINT4_G32 ? (const uint16_t*)(c->w + e.zp_offset) : nullptr;
  m.rows = (int32_t)e.rows;
  return m;
}

const float* gainp(const dec_ctx* c, int idx) { return (const float*)(c->w + c->blob.e[idx].offset); }

#define HIPCHECK(expr)                                                                        \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(&ctx->err, DEC_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// Pack the call's metadata into a pinned slot, upload it, and describe it for the kernels.
// `base` / `ws`: the scratch memory of the call (the workspace, or the static scratch) and its layout.
int upload_meta(dec_ctx* ctx, uint8_t* base, const Ws& ws, hipStream_t st, int32_t S, const int32_t* start,
                const int32_t* n_new, const int32_t* tokens, const int32_t* tables, int32_t max_blocks, int32_t mode,
                BatchDev* b, int* max_ctx) {
  const dec_config& c = ctx->cfg;
  int32_t N = 0, stride = 1, mc = 0;
  for (int s = 0; s < S; ++s) {
    const int32_t n = n_new ? n_new[s] : 1;
    N += n;
    stride = std::max<int32_t>(stride, (start[s] + n + c.block_tokens - 1) / c.block_tokens);
    mc = std::max<int32_t>(mc, start[s] + n);
  }
  const int32_t n_out = mode == DEC_LOGITS_ALL ? N : (mode == DEC_LOGITS_LAST ? S : 0);
  constexpr int QT = kPrefillQueryTile;
  int32_t n_tiles = 0;
  for (int s = 0; s < S; ++s) n_tiles += ((n_new ? n_new[s] : 1) + QT - 1) / QT;
  const size_t o_tok = 0, o_pos = N, o_seq = 2 * (size_t)N, o_sst = 3 * (size_t)N, o_snn = o_sst + S,
               o_sr0 = o_snn + S, o_out = o_sr0 + S, o_til = o_out + n_out, o_tbl = o_til + 2 * (size_t)n_tiles;
  // decode attention work items: only when a row has more keys than one segment takes
  const int32_t sk = ws.seg_keys;
  int32_t n_items = 0;
  if (!n_new) {
    bool split = false;
    for (int s = 0; s < S; ++s) split |= start[s] > sk;
    if (split)
      for (int s = 0; s < S; ++s) n_items += start[s] > sk ? (start[s] + sk - 1) / sk : 1;
  }
  const size_t o_itm = (o_tbl + (size_t)S * stride + 3) & ~(size_t)3;  // 16-byte aligned
  const size_t total = o_itm + 4 * (size_t)n_items;
  if (total > ws.meta_ints) return fail(&ctx->err, DEC_E_CAPACITY, "call metadata exceeds the workspace");

  const int slot = ctx->slot;
  ctx->slot = (slot + 1) % kSlots;
  HIPCHECK(hipEventSynchronize(ctx->ev[slot]));  // the slot's previous upload has finished
  int32_t* m = ctx->staging[slot];
  int32_t r = 0, t = 0;
  for (int s = 0; s < S; ++s) {
    const int32_t n = n_new ? n_new[s] : 1;
    m[o_sst + s] = start[s];
    m[o_snn + s] = n;
    m[o_sr0 + s] = r;
    for (int32_t i = 0; i < n; ++i, ++r) {
      m[o_tok + r] = tokens ? tokens[r] : 0;
      m[o_pos + r] = start[s] + i;
      m[o_seq + r] = s;
      if (mode == DEC_LOGITS_ALL) m[o_out + r] = r;
    }
    if (mode == DEC_LOGITS_LAST) m[o_out + s] = r - 1;
    for (int32_t i = 0; i < n; i += QT, ++t) {
      m[o_til + 2 * t] = s;
      m[o_til + 2 * t + 1] = m[o_sr0 + s] + i;
    }
    const int32_t need = (start[s] + n + c.block_tokens - 1) / c.block_tokens;
    for (int32_t j = 0; j < stride; ++j) m[o_tbl + (size_t)s * stride + j] = j < need ? tables[(size_t)s * max_blocks + j] : 0;
  }
  // attention tiles: sequence by sequence, each sequence's tiles from the last (most keys) to
  // the first, so that blocks running side by side share a sequence's keys in L2
  if (n_tiles > 1) {
    int32_t t2 = 0;
    for (int s = 0; s < S; ++s) {
      const int32_t n = n_new ? n_new[s] : 1, nt = (n + QT - 1) / QT;
      for (int32_t i = nt - 1; i >= 0; --i, ++t2) {
        m[o_til + 2 * t2] = s;
        m[o_til + 2 * t2 + 1] = m[o_sr0 + s] + i * QT;
      }
    }
  }
  if (n_items) {
    // (row, segment) items ordered by their key count, largest first (ties: row, then segment
    // order), so that the short items fill in at the end; each carries its row's position and
    // sequence (decode row s is sequence s), so a workgroup needs one load to start
    std::vector<std::pair<int32_t, int32_t>> it;  // (keys, row * 4096 + segment)
    it.reserve(n_items);
    for (int s = 0; s < S; ++s) {
      const int32_t ns = start[s] > sk ? (start[s] + sk - 1) / sk : 1;
      for (int32_t g = 0; g < ns; ++g) it.emplace_back(ns > 1 ? std::min(sk, start[s] - g * sk) : start[s], s * 4096 + g);
    }
    std::stable_sort(it.begin(), it.end(), [](const auto& x, const auto& y) { return x.first > y.first; });
    for (int32_t i = 0; i < n_items; ++i) {
      const int32_t s = it[i].second / 4096;
      int32_t* e = m + o_itm + 4 * (size_t)i;
      e[0] = s;
      e[1] = it[i].second % 4096;
      e[2] = start[s];
      e[3] = s;
    }
  }
  int32_t* dm = (int32_t*)(base + ws.meta);
  HIPCHECK(hipMemcpyAsync(dm, m, total * 4, hipMemcpyHostToDevice, st));
  HIPCHECK(hipEventRecord(ctx->ev[slot], st));
  b->row_tok = dm + o_tok;
  b->row_pos = dm + o_pos;
  b->row_seq = dm + o_seq;
  b->seq_start = dm + o_sst;
  b->seq_nnew = dm + o_snn;
  b->seq_row0 = dm + o_sr0;
  b->out_rows = dm + o_out;
  b->tiles = dm + o_til;
  b->block_tables = dm + o_tbl;
  b->dec_items = dm + o_itm;
  b->n_dec_items = n_items;
  b->seg_keys = sk;
  b->tbl_stride = stride;
  b->n_rows = N;
  b->n_seqs = S;
  b->n_out = n_out;
  b->n_tiles = n_tiles;
  *max_ctx = mc;
  return DEC_OK;
}

}  // namespace

LaunchTiming& dec::launch_timing() {
  static thread_local LaunchTiming t;
  return t;
}

namespace {

hipEvent_t timing_event(dec_ctx* ctx) {
  if (!ctx->timing.pool.empty()) {
    hipEvent_t e = ctx->timing.pool.back();
    ctx->timing.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Start of a timed launch: take two events, record the first on the stream and hand both to
// the launcher, which records them at the kernel's own start and end when it launches through
// launch_kernel (the later record supersedes the first). Returns false when the class is not
// timed.
bool timing_begin(dec_ctx* ctx, int cls, hipStream_t st, hipEvent_t* start, hipEvent_t* stop) {
  if (!(ctx->timing.mask & (1u << cls))) return false;
  *start = timing_event(ctx);
  *stop = *start ? timing_event(ctx) : nullptr;
  if (!*stop) return false;
  (void)hipEventRecord(*start, st);
  launch_timing() = LaunchTiming{*start, *stop, false};
  return true;
}

// End of a timed launch: a launcher that did not take the events gets the stop recorded after it.
void timing_end(dec_ctx* ctx, int cls, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  LaunchTiming& lt = launch_timing();
  if (!lt.used) (void)hipEventRecord(stop, st);
  lt = LaunchTiming{};
  ctx->timing.rec[cls].push_back({start, stop});
}

#define LAUNCH(expr)                                                                               \
  do {                                                                                             \
    hipError_t e_ = (expr);                                                                        \
    if (e_ != hipSuccess) return fail(&ctx->err, DEC_E_HIP, "launch %s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// A launch of kernel class `cls`, bracketed by events when that class is timed.
#define TLAUNCH(cls, expr)                                         \
  do {                                                             \
    hipEvent_t t0_ = nullptr, t1_ = nullptr;                       \
    const bool timed_ = timing_begin(ctx, cls, st, &t0_, &t1_);    \
    LAUNCH(expr);                                                  \
    if (timed_) timing_end(ctx, cls, st, t0_, t1_);                \
  } while (0)

// The forward pass over the uploaded batch: embedding, layers, final norm + LM head, argmax.
int run_forward(dec_ctx* ctx, uint8_t* base, const Ws& w, hipStream_t st, const BatchDev& b, const int32_t* tok_dev,
                int max_ctx, bool decode, float* logits, int32_t* next) {
  const dec_config& c = ctx->cfg;
  const int N = b.n_rows, d = c.d_model, H = c.n_heads, Hkv = c.n_kv_heads, D = c.head_dim;
  const int qw = H * D, qkvw = qw + 2 * Hkv * D, ff = c.ff_hidden;
  const bool act_bf16 = c.weight_dtype != DEC_F32;
  const bool kv_f16 = c.kv_dtype == DEC_F16;
  float* x = (float*)(base + w.x);
  void* h = base + w.h;
  float* qkv = (float*)(base + w.qkv);
  void* q = base + w.q;
  void* o = base + w.o;
  void* act = base + w.a;
  float* part = (float*)(base + w.part);
  float* dpart = (float*)(base + w.dpart);
  float* ssq = (float*)(base + w.ssq);
  uint16_t* xg = (uint16_t*)(base + w.xg);
  const float2* rope = (const float2*)(ctx->wsp + ctx->ws.rope);
  PoolDev pool{ctx->pool, c.n_blocks, Hkv, c.block_tokens, D, __builtin_ctz((unsigned)c.block_tokens)};
  const int nch = (max_ctx + w.chunk - 1) / w.chunk;
  // Decode steps take the decode GEMM (K split inside a block) when the weight format has one.
  // Its RMSNorm is deferred: the embedding and the residual epilogues write, beside x, the
  // residual's 16-column sums of squares and xg = bf16(x * g) with the gain g of the norm that
  // reads x next; the normalising products take xg as their input and scale each output row
  // by 1 / rms(x), so decode needs no separate RMSNorm launch. Prefill calls take the tile
  // GEMMs after an RMSNorm, launched on its own or (float32 residual products split over K)
  // written by the product's combine.
  const bool dgemm = decode && gemm_decode_supported(c.weight_dtype, d) &&
                     gemm_decode_supported(c.weight_dtype, qw) && gemm_decode_supported(c.weight_dtype, ff);
  // Prefill calls with bf16 / uint4 weights take the 256 x 256 tile GEMM, which also applies
  // the q/k norm, RoPE and the KV write in its Q|K|V epilogue (chosen by the configuration
  // alone, so every prefill call of a model computes the same way).
  // The other products take it when it fills the chip (>= 256 tiles, M >= 1024; SwiGLU with
  // bf16 weights: >= 512 tiles, two rounds of blocks), else (bf16 weights) its 128 x 128 form
  // when that fills the chip, else the 64 x 64 tiles; all give identical results, so the
  // choice never changes a row's bits.
  const bool big = !decode && gemm_big_supported(c.weight_dtype, EPI_QKV, D);
  // 4-bit weights, prefill calls of at least kWidenRows rows: each layer's matrices are first
  // widened to bf16 in the workspace (the values the 4-bit kernels stage as MFMA operands) and
  // the layer's products take the bf16 kernels, with identical results
  const bool widen = big && is_q4(c.weight_dtype) && w.wide_bytes > 0 && N >= kWidenRows;
  const int lwf = widen ? DEC_BF16 : c.weight_dtype;  // format of the layers' matrices as the products read them
  auto gemm = [&](int epi, const GemmArgs& g0, int wf) {
    if (dgemm) return launch_gemm_decode(wf, epi, g0, st);
    GemmArgs g = g0;
    g.part = (float*)(base + w.fpart);
    g.part_floats = (int64_t)w.fpart_floats;
    auto tiles = [&](int t) {
      return (g.M + t - 1) / t * (epi == EPI_SWIGLU ? (g.N + t / 2 - 1) / (t / 2) : (g.N + t - 1) / t);
    };
    const bool mid = big && gemm_mid_supported(wf, epi) && tiles(128) >= 256;
    const int big_min = mid && epi == EPI_SWIGLU ? 512 : 256;
    if (big && tiles(256) >= big_min && g.M >= 1024) return launch_gemm_big(wf, epi, g, nullptr, st);
    if (mid) return launch_gemm_mid(wf, epi, g, st);
    return launch_gemm(wf, epi, g, st);
  };
  // Float32 residual products that split K over blocks write the next RMSNorm's output h
  // themselves, in their combine (same arithmetic as the norm launch): set the product's norm
  // arguments when it does, and report whether it does
  auto fuse_norm = [&](GemmArgs& g0, int wf, const float* gain) {
    if (dgemm || big || act_bf16) return false;
    GemmArgs t = g0;
    t.part = (float*)(base + w.fpart);
    t.part_floats = (int64_t)w.fpart_floats;
    t.norm_g = gain;
    t.norm_out = (float*)h;
    t.norm_eps = c.rms_eps;
    if (!gemm_fuses_norm(wf, EPI_RESID, t)) return false;
    g0.norm_g = t.norm_g;
    g0.norm_out = t.norm_out;
    g0.norm_eps = t.norm_eps;
    return true;
  };
  // A of a normalising GEMM: the residual itself (decode GEMM) or the RMSNorm output
  // (gain: the norm's gain, applied to xg by the product that wrote it)
  auto norm_input = [&](GemmArgs& g, const float* gain) {
    (void)gain;
    if (dgemm) {
      g.A = xg; g.lda = d; g.ssq_in = ssq; g.eps = c.rms_eps;
    } else {
      g.A = h; g.lda = d;
    }
  };

  TLAUNCH(DEC_K_EMBED, launch_embed(tok_dev ? tok_dev : b.row_tok, N, c.vocab, d, c.weight_dtype, ctx->embed, x,
                                    dgemm ? ssq : nullptr, dgemm ? xg : nullptr, ctx->layers[0].attn_norm, st));
  bool h_ready = false;  // h already holds this layer's attention-norm output (fused above)
  for (int l = 0; l < c.n_layers; ++l) {
    LayerW Lw;
    if (widen) {
      // the layer's seven matrices, one after another in the widened region
      const LayerW& L0 = ctx->layers[l];
      uint16_t* wb = (uint16_t*)(base + w.wide);
      const WMat src[7] = {L0.wq, L0.wk, L0.wv, L0.wo, L0.wg, L0.wu, L0.wd};
      const int cols[7] = {d, d, d, qw, d, d, ff};
      WMat* dst[7] = {&Lw.wq, &Lw.wk, &Lw.wv, &Lw.wo, &Lw.wg, &Lw.wu, &Lw.wd};
      int64_t offs[7], o = 0;
      Lw = L0;
      for (int j = 0; j < 7; ++j) {
        offs[j] = o;
        *dst[j] = WMat{wb + o, nullptr, nullptr, src[j].rows};
        o += (int64_t)src[j].rows * cols[j];
      }
      TLAUNCH(DEC_K_WIDEN, launch_widen_q4(c.weight_dtype, src, cols, offs, 7, wb, st));
    }
    const LayerW& L = widen ? Lw : ctx->layers[l];
    if (!dgemm && !h_ready)
      TLAUNCH(DEC_K_RMSNORM, launch_rmsnorm(x, nullptr, N, d, L.attn_norm, c.rms_eps, h, act_bf16, st));
    h_ready = false;
    GemmArgs g{};
    norm_input(g, L.attn_norm);
    g.M = N; g.N = qkvw; g.K = d;
    g.seg[0] = L.wq; g.seg[1] = L.wk; g.seg[2] = L.wv; g.nseg = 3;
    g.C = qkv; g.ldc = qkvw;
    QkRopeArgs qa{qkv, L.q_norm, L.k_norm, rope, q, pool, l, H, Hkv, D, c.rms_eps, kv_f16, b};
    bool qk_done = false;  // the product's combine did the q/k norm, RoPE and K/V write
    if (big) {
      TLAUNCH(DEC_K_GEMM_QKV, launch_gemm_big(lwf, EPI_QKV, g, &qa, st));
    } else {
      if (!decode && !dgemm) {
        GemmArgs t = g;
        t.part = (float*)(base + w.fpart);
        t.part_floats = (int64_t)w.fpart_floats;
        t.qk = &qa;
        qk_done = gemm_fuses_qk(lwf, EPI_STORE, t);
        if (qk_done) g.qk = &qa;
      }
      TLAUNCH(DEC_K_GEMM_QKV, gemm(EPI_STORE, g, lwf));
    }
    if (decode) {
      AttnRowsArgs ra{q, pool, l, H, Hkv, D, kv_f16, w.dslots, dpart, b};
      TLAUNCH(DEC_K_ATTN_ROWS, launch_attn_decode(qa, ra, o, act_bf16, st));
      if (b.n_dec_items) TLAUNCH(DEC_K_ATTN_COMBINE, launch_attn_decode_combine(ra, o, act_bf16, st));
    } else {
      if (!big && !qk_done) TLAUNCH(DEC_K_QK_ROPE_KV, launch_qk_rope_kv(qa, st));
      if (w.flash) {
        AttnPrefillArgs pa{(const uint16_t*)q, pool, l, H, Hkv, D, o, act_bf16, b};
        TLAUNCH(DEC_K_ATTN_PREFILL, launch_attn_prefill(pa, st));
      } else {
        AttnRowsArgs ra{q, pool, l, H, Hkv, D, kv_f16, nch, part, b};
        if (nch <= attn_rows_merged_max_chunks(D, H / Hkv)) {
          TLAUNCH(DEC_K_ATTN_ROWS, launch_attn_rows_merged(ra, o, act_bf16, st));
        } else {
          TLAUNCH(DEC_K_ATTN_ROWS, launch_attn_rows(ra, st));
          TLAUNCH(DEC_K_ATTN_COMBINE, launch_attn_combine(part, N, H, D, nch, w.chunk, b.row_pos, o, act_bf16, st));
        }
      }
    }
    g = GemmArgs{};
    g.A = o; g.lda = qw; g.M = N; g.N = d; g.K = qw;
    g.seg[0] = L.wo; g.nseg = 1; g.C = x; g.ldc = d;
    g.ssq_out = dgemm ? ssq : nullptr;
    g.xg_out = dgemm ? xg : nullptr; g.gain_next = L.ffn_norm;
    const bool o_norm = fuse_norm(g, lwf, L.ffn_norm);
    TLAUNCH(DEC_K_GEMM_O, gemm(EPI_RESID, g, lwf));
    if (!dgemm && !o_norm)
      TLAUNCH(DEC_K_RMSNORM, launch_rmsnorm(x, nullptr, N, d, L.ffn_norm, c.rms_eps, h, act_bf16, st));
    g = GemmArgs{};
    norm_input(g, L.ffn_norm);
    g.M = N; g.N = ff; g.K = d;
    g.seg[0] = L.wg; g.seg[1] = L.wu; g.nseg = 2; g.C = act; g.ldc = ff; g.c_bf16 = act_bf16;
    TLAUNCH(DEC_K_GEMM_GATEUP, gemm(EPI_SWIGLU, g, lwf));
    g = GemmArgs{};
    g.A = act; g.lda = ff; g.M = N; g.N = d; g.K = ff;
    g.seg[0] = L.wd; g.nseg = 1; g.C = x; g.ldc = d;
    g.ssq_out = dgemm ? ssq : nullptr;
    g.xg_out = dgemm ? xg : nullptr;
    g.gain_next = l + 1 < c.n_layers ? ctx->layers[l + 1].attn_norm : ctx->final_norm;
    if (l + 1 < c.n_layers) h_ready = fuse_norm(g, lwf, ctx->layers[l + 1].attn_norm);
    TLAUNCH(DEC_K_GEMM_DOWN, gemm(EPI_RESID, g, lwf));
  }
  if (b.n_out > 0 && logits) {
    GemmArgs g{};
    if (dgemm) {
      // decode: every row gets logits, in row order (one row per sequence)
      norm_input(g, ctx->final_norm);
    } else {
      TLAUNCH(DEC_K_RMSNORM, launch_rmsnorm(x, b.out_rows, b.n_out, d, ctx->final_norm, c.rms_eps, h, act_bf16, st));
      g.A = h; g.lda = d;
    }
    g.M = b.n_out; g.N = c.vocab; g.K = d;
    g.seg[0] = ctx->embed; g.nseg = 1; g.C = logits; g.ldc = c.vocab;
    // decode with greedy ids: the LM head writes per-block candidates and one pass picks them
    const int cand = dgemm && next && lmhead_decode_supported(c.weight_dtype, b.n_out, d)
                         ? lmhead_decode_parts(b.n_out, c.vocab)
                         : 0;
    float* cand_v = (float*)(base + w.amax);
    int32_t* cand_i = (int32_t*)(cand_v + (size_t)b.n_out * std::max(cand, 1));
    if (cand) {
      g.am_v = cand_v;
      g.am_i = cand_i;
    }
    if (dgemm && lmhead_decode_supported(c.weight_dtype, b.n_out, d)) {
      TLAUNCH(DEC_K_GEMM_LMHEAD, launch_lmhead_decode(c.weight_dtype, g, st));
    } else {
      TLAUNCH(DEC_K_GEMM_LMHEAD, gemm(EPI_STORE, g, c.weight_dtype));
    }
    if (next && cand) {
      TLAUNCH(DEC_K_ARGMAX, launch_argmax_final(cand_v, cand_i, b.n_out, cand, next, st));
    } else if (next) {
      TLAUNCH(DEC_K_ARGMAX, launch_argmax(logits, b.n_out, c.vocab, next, base + w.amax, st));
    }
  }
  return DEC_OK;
}

}  // namespace

namespace {

// A decode step with its per-call scratch at `base` (layout `ws`); checks as dec_decode_step.
int decode_step(dec_ctx* ctx, uint8_t* base, const Ws* ws, void* stream, int32_t n_seqs, const int32_t* tokens_host,
                const int32_t* tokens_device, const int32_t* positions, const int32_t* block_tables, int32_t max_blocks,
                float* logits, int32_t* next_tokens) {
  if ((tokens_host == nullptr) == (tokens_device == nullptr))
    return fail(&ctx->err, DEC_E_ARG, "exactly one of tokens_host and tokens_device must be given");
  if (next_tokens && !logits) return fail(&ctx->err, DEC_E_ARG, "next_tokens needs logits");
  const int mode = logits ? DEC_LOGITS_LAST : DEC_LOGITS_NONE;
  int rc = check_step(ctx->cfg, n_seqs, positions, nullptr, tokens_host, block_tables, max_blocks, mode, &ctx->err);
  if (rc) return rc;
  Ws lw;
  if (!ws) {  // the static scratch, laid out for this call's sequences
    lw = ws_layout(ctx->cfg, n_seqs);
    if (lw.total > kStaticScratchBytes)
      return fail(&ctx->err, DEC_E_CAPACITY,
                  "a decode step of %d sequences needs %zu bytes of scratch, above the %zu bytes of the static scratch",
                  n_seqs, lw.total, kStaticScratchBytes);
    if (!base) return fail(&ctx->err, DEC_E_HIP, "the static scratch's device address is unknown: %s", ctx->scratch_err.c_str());
    ws = &lw;
  }
  hipStream_t st = (hipStream_t)stream;
  BatchDev b{};
  int max_ctx = 0;
  rc = upload_meta(ctx, base, *ws, st, n_seqs, positions, nullptr, tokens_host, block_tables, max_blocks, mode, &b,
                   &max_ctx);
  if (rc) return rc;
  return run_forward(ctx, base, *ws, st, b, tokens_device, max_ctx, true, logits, next_tokens);
}

}  // namespace

extern "C" {

int dec_check_config(const dec_config* cfg) { return check_config(cfg, &g_err); }

size_t dec_weight_bytes(const dec_config* cfg) {
  if (check_config(cfg, &g_err)) return 0;
  return blob_layout(*cfg).total;
}

int dec_weight_count(const dec_config* cfg) {
  if (check_config(cfg, &g_err)) return 0;
  return 2 + kPerLayer * cfg->n_layers;
}

int dec_weight_entry(const dec_config* cfg, int index, dec_weight_info* out) {
  int rc = check_config(cfg, &g_err);
  if (rc) return rc;
  if (!out) return fail(&g_err, DEC_E_ARG, "out is NULL");
  Blob b = blob_layout(*cfg);
  if (index < 0 || index >= (int)b.e.size()) return fail(&g_err, DEC_E_ARG, "entry index %d out of range", index);
  *out = b.e[index];
  return DEC_OK;
}

size_t dec_kv_pool_bytes(const dec_config* cfg) {
  if (check_config(cfg, &g_err)) return 0;
  return kv_bytes(*cfg);
}

size_t dec_workspace_bytes(const dec_config* cfg) {
  if (check_config(cfg, &g_err)) return 0;
  return ws_layout(*cfg).total;
}

int dec_check_step(const dec_config* cfg, int32_t n_seqs, const int32_t* start, const int32_t* n_new,
                   const int32_t* tokens, const int32_t* block_tables, int32_t max_blocks, int32_t logits_mode,
                   char* msg, size_t msg_len) {
  std::string err;
  int rc = check_config(cfg, &err);
  if (!rc) rc = check_step(*cfg, n_seqs, start, n_new, tokens, block_tables, max_blocks, logits_mode, &err);
  if (msg && msg_len) snprintf(msg, msg_len, "%s", rc ? err.c_str() : "");
  return rc;
}

const char* dec_last_error(const dec_ctx* ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

int dec_init(const dec_config* cfg, const void* weights, size_t weight_bytes, void* kv_pool, size_t kv_bytes_in,
             void* workspace, size_t workspace_bytes, void* stream, dec_ctx** out) {
  if (!out) return fail(&g_err, DEC_E_ARG, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg, &g_err);
  if (rc) return rc;
  if (!weights || !kv_pool || !workspace) return fail(&g_err, DEC_E_ARG, "weights, kv_pool and workspace must be non-NULL");
  if (((uintptr_t)weights | (uintptr_t)kv_pool | (uintptr_t)workspace) % kAlign)
    return fail(&g_err, DEC_E_ARG, "weights, kv_pool and workspace must be 256-byte aligned");
  dec_ctx* ctx = new dec_ctx();
  ctx->cfg = *cfg;
  ctx->blob = blob_layout(*cfg);
  ctx->ws = ws_layout(*cfg);
  if (weight_bytes < ctx->blob.total || kv_bytes_in < kv_bytes(*cfg) || workspace_bytes < ctx->ws.total) {
    rc = fail(&g_err, DEC_E_CAPACITY, "buffers too small: weights %zu < %zu, kv %zu < %zu or workspace %zu < %zu",
              weight_bytes, ctx->blob.total, kv_bytes_in, kv_bytes(*cfg), workspace_bytes, ctx->ws.total);
    delete ctx;
    return rc;
  }
  ctx->w = (const uint8_t*)weights;
  ctx->pool = kv_pool;
  ctx->wsp = (uint8_t*)workspace;
  ctx->slot = 0;
  for (int i = 0; i < kSlots; ++i) {
    ctx->staging[i] = nullptr;
    ctx->ev[i] = nullptr;
  }
  ctx->samp_staging = nullptr;
  ctx->samp_ev = nullptr;
  ctx->scratch = static_scratch(&ctx->scratch_err);  // (with the ctx's device current)
  ctx->embed = wmat(ctx, 0);
  for (int l = 0; l < cfg->n_layers; ++l) {
    const int b = 1 + l * kPerLayer;
    LayerW L;
    L.attn_norm = gainp(ctx, b + 0);
    L.wq = wmat(ctx, b + 1);
    L.wk = wmat(ctx, b + 2);
    L.wv = wmat(ctx, b + 3);
    L.q_norm = gainp(ctx, b + 4);
    L.k_norm = gainp(ctx, b + 5);
    L.wo = wmat(ctx, b + 6);
    L.ffn_norm = gainp(ctx, b + 7);
    L.wg = wmat(ctx, b + 8);
    L.wu = wmat(ctx, b + 9);
    L.wd = wmat(ctx, b + 10);
    ctx->layers.push_back(L);
  }
  ctx->final_norm = gainp(ctx, 1 + cfg->n_layers * kPerLayer);

  hipStream_t st = (hipStream_t)stream;
  auto bail = [&](hipError_t e, const char* what) {
    rc = fail(&g_err, DEC_E_HIP, "%s: %s", what, hipGetErrorString(e));
    dec_free(ctx);
    return rc;
  };
  for (int i = 0; i < kSlots; ++i) {
    hipError_t e = hipHostMalloc((void**)&ctx->staging[i], ctx->ws.meta_ints * 4, hipHostMallocDefault);
    if (e != hipSuccess) return bail(e, "hipHostMalloc");
    e = hipEventCreateWithFlags(&ctx->ev[i], hipEventDisableTiming);
    if (e != hipSuccess) return bail(e, "hipEventCreate");
  }
  {
    hipError_t e = hipHostMalloc((void**)&ctx->samp_staging, (size_t)cfg->max_seqs * sizeof(SampleSeq),
                                 hipHostMallocDefault);
    if (e != hipSuccess) return bail(e, "hipHostMalloc");
    e = hipEventCreateWithFlags(&ctx->samp_ev, hipEventDisableTiming);
    if (e != hipSuccess) return bail(e, "hipEventCreate");
    // the sampler's count table starts zero; every dec_sample call leaves it zero
    e = hipMemsetAsync(ctx->wsp + ctx->ws.counts, 0, (size_t)cfg->max_seqs * cfg->vocab * 4, st);
    if (e != hipSuccess) return bail(e, "hipMemsetAsync(counts)");
  }
  // RoPE table: angle p * base^(-2j/D) in double precision, cos/sin rounded once to float
  const int half = cfg->head_dim / 2;
  std::vector<float2> rope((size_t)cfg->max_context * half);
  for (int j = 0; j < half; ++j) {
    const double inv = std::pow(cfg->rope_base, -2.0 * j / cfg->head_dim);
    for (int p = 0; p < cfg->max_context; ++p) {
      const double ang = (double)p * inv;
      rope[(size_t)p * half + j] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  }
  hipError_t e = hipMemcpyAsync(ctx->wsp + ctx->ws.rope, rope.data(), rope.size() * sizeof(float2),
                                hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return bail(e, "hipMemcpyAsync(rope)");
  e = hipStreamSynchronize(st);  // the host copy of the table goes out of scope
  if (e != hipSuccess) return bail(e, "hipStreamSynchronize");
  *out = ctx;
  return DEC_OK;
}

int dec_timing_enable(dec_ctx* ctx, uint32_t class_mask) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  ctx->timing.mask = class_mask & ((1u << DEC_K_COUNT) - 1);
  return DEC_OK;
}

int dec_timing_read(dec_ctx* ctx, int kernel_class, double* total_ms, int64_t* launches) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  if (kernel_class < 0 || kernel_class >= DEC_K_COUNT) return fail(&ctx->err, DEC_E_ARG, "unknown kernel class");
  double total = 0.0;
  auto& rec = ctx->timing.rec[kernel_class];
  for (auto& pr : rec) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(pr.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) return fail(&ctx->err, DEC_E_HIP, "timing events: %s", hipGetErrorString(e));
    total += ms;
    ctx->timing.pool.push_back(pr.first);
    ctx->timing.pool.push_back(pr.second);
  }
  if (total_ms) *total_ms = total;
  if (launches) *launches = (int64_t)rec.size();
  rec.clear();
  return DEC_OK;
}

void dec_free(dec_ctx* ctx) {
  if (!ctx) return;
  for (auto& rec : ctx->timing.rec)
    for (auto& pr : rec) {
      (void)hipEventSynchronize(pr.second);
      ctx->timing.pool.push_back(pr.first);
      ctx->timing.pool.push_back(pr.second);
    }
  for (hipEvent_t e : ctx->timing.pool) (void)hipEventDestroy(e);
  for (int i = 0; i < kSlots; ++i) {
    if (ctx->ev[i]) {
      (void)hipEventSynchronize(ctx->ev[i]);
      (void)hipEventDestroy(ctx->ev[i]);
    }
    if (ctx->staging[i]) (void)hipHostFree(ctx->staging[i]);
  }
  if (ctx->samp_ev) {
    (void)hipEventSynchronize(ctx->samp_ev);
    (void)hipEventDestroy(ctx->samp_ev);
  }
  if (ctx->samp_staging) (void)hipHostFree(ctx->samp_staging);
  delete ctx;
}

int dec_prefill(dec_ctx* ctx, void* stream, int32_t n_seqs, const int32_t* start, const int32_t* n_new,
                const int32_t* tokens, const int32_t* block_tables, int32_t max_blocks, int32_t logits_mode,
                float* logits, int32_t* next_tokens) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  if (!n_new) return fail(&ctx->err, DEC_E_ARG, "n_new is NULL");
  if (!tokens) return fail(&ctx->err, DEC_E_ARG, "tokens is NULL");
  int rc = check_step(ctx->cfg, n_seqs, start, n_new, tokens, block_tables, max_blocks, logits_mode, &ctx->err);
  if (rc) return rc;
  if (logits_mode != DEC_LOGITS_NONE && !logits) return fail(&ctx->err, DEC_E_ARG, "logits is NULL");
  if (next_tokens && logits_mode == DEC_LOGITS_NONE) return fail(&ctx->err, DEC_E_ARG, "next_tokens needs logits");
  hipStream_t st = (hipStream_t)stream;
  BatchDev b{};
  int max_ctx = 0;
  rc = upload_meta(ctx, ctx->wsp, ctx->ws, st, n_seqs, start, n_new, tokens, block_tables, max_blocks, logits_mode, &b,
                   &max_ctx);
  if (rc) return rc;
  return run_forward(ctx, ctx->wsp, ctx->ws, st, b, nullptr, max_ctx, false,
                     logits_mode == DEC_LOGITS_NONE ? nullptr : logits, next_tokens);
}


int dec_decode_step(dec_ctx* ctx, void* stream, int32_t n_seqs, const int32_t* tokens_host,
                    const int32_t* tokens_device, const int32_t* positions, const int32_t* block_tables,
                    int32_t max_blocks, float* logits, int32_t* next_tokens) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  return decode_step(ctx, ctx->wsp, &ctx->ws, stream, n_seqs, tokens_host, tokens_device, positions, block_tables,
                     max_blocks, logits, next_tokens);
}

int dec_decode_step_static(dec_ctx* ctx, void* stream, int32_t n_seqs, const int32_t* tokens_host,
                           const int32_t* tokens_device, const int32_t* positions, const int32_t* block_tables,
                           int32_t max_blocks, float* logits, int32_t* next_tokens) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  return decode_step(ctx, (uint8_t*)ctx->scratch, nullptr, stream, n_seqs, tokens_host, tokens_device, positions,
                     block_tables, max_blocks, logits, next_tokens);
}

void dec_rng_stream(uint64_t seed, uint64_t purpose, uint64_t state_inc[2]) {
  // child_seed = mix64(seed + purpose * golden gamma), mix64 the splitmix64 finaliser; then
  // pcg32_srandom_r(child_seed, purpose): inc = 2 purpose + 1, one step from state 0, add the
  // seed, one more step (the step's output is not needed here)
  uint64_t z = seed + purpose * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  const uint64_t inc = (purpose << 1) | 1u;
  uint64_t st = 0;
  st = st * 6364136223846793005ull + inc;
  st += z;
  st = st * 6364136223846793005ull + inc;
  state_inc[0] = st;
  state_inc[1] = inc;
}

int dec_sample(dec_ctx* ctx, void* stream, int32_t n_seqs, const float* logits, int64_t ld,
               const dec_sampling* params, const dec_history* history, const int32_t* ids, int64_t n_ids,
               uint64_t* rng, int32_t* next, double* logprob) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  const int V = ctx->cfg.vocab;
  if (n_seqs <= 0) return fail(&ctx->err, DEC_E_ARG, "n_seqs must be >= 1");
  if (n_seqs > ctx->cfg.max_seqs) return fail(&ctx->err, DEC_E_CAPACITY, "n_seqs %d exceeds max_seqs %d", n_seqs, ctx->cfg.max_seqs);
  if (!logits || !params || !history || !rng || !next) return fail(&ctx->err, DEC_E_ARG, "a required pointer is NULL");
  if (ld < V) return fail(&ctx->err, DEC_E_ARG, "ld %lld is below the vocabulary", (long long)ld);
  if (V > 262144) return fail(&ctx->err, DEC_E_UNSUPPORTED, "the sampler takes vocabularies up to 262,144 ids");
  if (n_ids < 0 || (n_ids > 0 && !ids)) return fail(&ctx->err, DEC_E_ARG, "ids is NULL or n_ids negative");
  for (int s = 0; s < n_seqs; ++s) {
    const dec_sampling& p = params[s];
    const dec_history& h = history[s];
    if (!(std::isfinite(p.temperature) && p.temperature >= 0.0)) return fail(&ctx->err, DEC_E_ARG, "sequence %d: temperature must be finite and >= 0", s);
    if (!(p.top_p > 0.0 && p.top_p <= 1.0)) return fail(&ctx->err, DEC_E_ARG, "sequence %d: top_p must be in (0, 1]", s);
    if (!(p.min_p >= 0.0 && p.min_p <= 1.0)) return fail(&ctx->err, DEC_E_ARG, "sequence %d: min_p must be in [0, 1]", s);
    if (!(std::isfinite(p.repetition_penalty) && p.repetition_penalty > 0.0))
      return fail(&ctx->err, DEC_E_ARG, "sequence %d: repetition_penalty must be finite and > 0", s);
    if (!std::isfinite(p.presence_penalty) || !std::isfinite(p.frequency_penalty))
      return fail(&ctx->err, DEC_E_ARG, "sequence %d: presence and frequency penalties must be finite", s);
    if (p.top_k < 0 || p.reserved != 0) return fail(&ctx->err, DEC_E_ARG, "sequence %d: top_k must be >= 0, reserved 0", s);
    if (h.prompt_offset < 0 || h.prompt_len < 0 || (int64_t)h.prompt_offset + h.prompt_len > n_ids ||
        h.output_offset < 0 || h.output_len < 0 || (int64_t)h.output_offset + h.output_len > n_ids)
      return fail(&ctx->err, DEC_E_ARG, "sequence %d: history ranges outside the id array", s);
  }
  hipStream_t st = (hipStream_t)stream;
  HIPCHECK(hipEventSynchronize(ctx->samp_ev));  // the previous call's upload has finished
  for (int s = 0; s < n_seqs; ++s) {
    ctx->samp_staging[s].p = params[s];
    ctx->samp_staging[s].h = history[s];
  }
  SampleSeq* dseq = (SampleSeq*)(ctx->wsp + ctx->ws.samp);
  HIPCHECK(hipMemcpyAsync(dseq, ctx->samp_staging, (size_t)n_seqs * sizeof(SampleSeq), hipMemcpyHostToDevice, st));
  HIPCHECK(hipEventRecord(ctx->samp_ev, st));
  LAUNCH(launch_sample(logits, ld, n_seqs, V, dseq, ids, (uint32_t*)(ctx->wsp + ctx->ws.counts), rng, next,
                       logprob, st));
  return DEC_OK;
}

// ---- export / import of blocks' K/V data ---------------------------------------------------
// Envelope: a header (magic "DECKVB01", n_layers, n_kv_heads, block_tokens, head_dim, kv_dtype,
// n blocks as int32), the n fills (int32), then per block and per layer its K slab and its V
// slab ([H_kv][B][D] of the KV dtype each).

namespace {
struct KvEnvHeader {
  char magic[8];
  int32_t n_layers, n_kv_heads, block_tokens, head_dim, kv_dtype, n;
};
size_t kv_slab_bytes(const dec_config& c) {
  return (size_t)c.n_kv_heads * c.block_tokens * c.head_dim * (c.kv_dtype == DEC_F16 ? 2 : 4);
}
}  // namespace

size_t dec_kv_export_bytes(const dec_ctx* ctx, int32_t n) {
  if (!ctx || n < 0) return 0;
  return sizeof(KvEnvHeader) + (size_t)n * 4 + (size_t)n * ctx->cfg.n_layers * 2 * kv_slab_bytes(ctx->cfg);
}

int dec_kv_export(dec_ctx* ctx, void* stream, const int32_t* ids, const int32_t* fills, int32_t n, void* buf,
                  size_t buf_bytes) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  const dec_config& c = ctx->cfg;
  if (n < 1 || !ids || !fills || !buf) return fail(&ctx->err, DEC_E_ARG, "export: NULL argument or n < 1");
  if (buf_bytes < dec_kv_export_bytes(ctx, n)) return fail(&ctx->err, DEC_E_CAPACITY, "export: buffer too small");
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= c.n_blocks) return fail(&ctx->err, DEC_E_BLOCK, "export: block id %d outside the pool", ids[i]);
    if (fills[i] < 0 || fills[i] > c.block_tokens) return fail(&ctx->err, DEC_E_ARG, "export: fill outside [0, block_tokens]");
  }
  KvEnvHeader h{};
  std::memcpy(h.magic, "DECKVB01", 8);
  h.n_layers = c.n_layers;
  h.n_kv_heads = c.n_kv_heads;
  h.block_tokens = c.block_tokens;
  h.head_dim = c.head_dim;
  h.kv_dtype = c.kv_dtype;
  h.n = n;
  uint8_t* out = (uint8_t*)buf;
  std::memcpy(out, &h, sizeof h);
  std::memcpy(out + sizeof h, fills, (size_t)n * 4);
  uint8_t* dst = out + sizeof h + (size_t)n * 4;
  const size_t sb = kv_slab_bytes(c);
  hipStream_t st = (hipStream_t)stream;
  for (int32_t i = 0; i < n; ++i)
    for (int l = 0; l < c.n_layers; ++l)
      for (int kv = 0; kv < 2; ++kv) {
        const uint8_t* src = (const uint8_t*)ctx->pool + (((size_t)l * 2 + kv) * c.n_blocks + ids[i]) * sb;
        HIPCHECK(hipMemcpyAsync(dst, src, sb, hipMemcpyDeviceToHost, st));
        dst += sb;
      }
  HIPCHECK(hipStreamSynchronize(st));
  return DEC_OK;
}

int dec_kv_import(dec_ctx* ctx, void* stream, const void* buf, size_t buf_bytes, const int32_t* ids, int32_t n,
                  int32_t* fills) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  const dec_config& c = ctx->cfg;
  if (!buf || !ids || n < 1) return fail(&ctx->err, DEC_E_ARG, "import: NULL argument or n < 1");
  KvEnvHeader h{};
  if (buf_bytes < sizeof h) return fail(&ctx->err, DEC_E_ARG, "import: buffer shorter than its header");
  std::memcpy(&h, buf, sizeof h);
  if (std::memcmp(h.magic, "DECKVB01", 8) != 0) return fail(&ctx->err, DEC_E_ARG, "import: not a KV block envelope");
  if (h.n_layers != c.n_layers || h.n_kv_heads != c.n_kv_heads || h.block_tokens != c.block_tokens ||
      h.head_dim != c.head_dim || h.kv_dtype != c.kv_dtype)
    return fail(&ctx->err, DEC_E_UNSUPPORTED, "import: the envelope's block format differs from this pool's");
  if (h.n != n) return fail(&ctx->err, DEC_E_ARG, "import: the envelope holds %d blocks, %d destinations given", h.n, n);
  if (buf_bytes != dec_kv_export_bytes(ctx, n)) return fail(&ctx->err, DEC_E_ARG, "import: buffer size does not match its header");
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c.n_blocks) return fail(&ctx->err, DEC_E_BLOCK, "import: block id %d outside the pool", ids[i]);
  const uint8_t* in = (const uint8_t*)buf + sizeof h;
  if (fills) std::memcpy(fills, in, (size_t)n * 4);
  const uint8_t* srcp = in + (size_t)n * 4;
  const size_t sb = kv_slab_bytes(c);
  hipStream_t st = (hipStream_t)stream;
  for (int32_t i = 0; i < n; ++i)
    for (int l = 0; l < c.n_layers; ++l)
      for (int kv = 0; kv < 2; ++kv) {
        uint8_t* dst = (uint8_t*)ctx->pool + (((size_t)l * 2 + kv) * c.n_blocks + ids[i]) * sb;
        HIPCHECK(hipMemcpyAsync(dst, srcp, sb, hipMemcpyHostToDevice, st));
        srcp += sb;
      }
  HIPCHECK(hipStreamSynchronize(st));  // the host buffer may be reused once this returns
  return DEC_OK;
}

int dec_quantize_int4_sym(void* stream, const float* w, int64_t rows, int64_t cols, uint8_t* q, uint16_t* scale) {
  if (!w || !q || !scale) return fail(&g_err, DEC_E_ARG, "quantize: NULL argument");
  if (rows < 1 || cols < 32 || cols % 32) return fail(&g_err, DEC_E_ARG, "quantize: rows >= 1, cols a positive multiple of 32");
  if (((uintptr_t)w | (uintptr_t)q) % 16) return fail(&g_err, DEC_E_ARG, "quantize: w and q must be 16-byte aligned");
  const hipError_t e = launch_quant_int4_sym(w, rows, cols, q, scale, (hipStream_t)stream);
  if (e != hipSuccess) return fail(&g_err, DEC_E_HIP, "quantize: %s", hipGetErrorString(e));
  return DEC_OK;
}

int dec_debug_dequant(dec_ctx* ctx, void* stream, int index, float* out) {
  if (!ctx) return fail(&g_err, DEC_E_ARG, "ctx is NULL");
  if (!out) return fail(&ctx->err, DEC_E_ARG, "out is NULL");
  if (index < 0 || index >= (int)ctx->blob.e.size()) return fail(&ctx->err, DEC_E_ARG, "entry index out of range");
  const dec_weight_info& e = ctx->blob.e[index];
  if (e.rows == 1 && e.dtype == DEC_F32 && std::strstr(e.name, "norm"))
    return fail(&ctx->err, DEC_E_ARG, "entry %d (%s) is a gain vector, not a matrix", index, e.name);
  LAUNCH(launch_dequant(e.dtype, wmat(ctx, index), (int)e.rows, (int)e.cols, out, (hipStream_t)stream));
  return DEC_OK;
}

}  // extern "C"
