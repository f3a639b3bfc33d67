// Launchers of the decoder kernels. All launch on the given stream and return
// the launch status; shapes are validated by the host runtime before any call.
#pragma once

#include <hip/hip_ext.h>

#include "common.h"

namespace dec {

constexpr int kPrefillQueryTile = 128;
// Decode attention splits a row with more than this many keys before its position (or more
// than one block of them, if blocks are larger) into segments of that many keys, one
// workgroup each; the split depends only on the row's own position.
constexpr int kDecodeSegKeys = 4096;
constexpr int kDecodeMaxSegs = 4095;  // segments per row (the host sorts items by row * 4096 + segment)

// Timed launches: while `start` is set and unused, the next kernel launched through
// launch_kernel records `start` and `stop` at its own dispatch begin and end (HIP's extended
// launch), so the measured duration is the kernel's alone, without the launch gap.
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
LaunchTiming& launch_timing();  // per host thread

template <typename... KA, typename... A>
inline void launch_kernel(void (*kernel)(KA...), dim3 g, dim3 b, uint32_t shmem, hipStream_t s, A... args) {
  LaunchTiming& t = launch_timing();
  if (t.start && !t.used) {
    hipExtLaunchKernelGGL(kernel, g, b, shmem, s, t.start, t.stop, 0u, args...);
    t.used = true;
  } else {
    kernel<<<g, b, shmem, s>>>(args...);
  }
}

// x[r][:] = widened/dequantised E[tok[r]][:] as float32; an id outside [0, vocab) gives NaN.
// ssq (optional, [n_rows][d/16]): sums of squares of each 16 columns of the row; with it, xg
// ([n_rows][d] bf16) receives x * g, the input of the first product's deferred RMSNorm.
hipError_t launch_embed(const int32_t* tok, int n_rows, int vocab, int d, int wdtype, const WMat& E,
                        float* x, float* ssq, uint16_t* xg, const float* g, hipStream_t s);

// out[r][:] = x[rows ? rows[r] : r][:] / sqrt(mean(x^2) + eps) * g, stored as float32 or bf16.
hipError_t launch_rmsnorm(const float* x, const int32_t* rows, int n, int d, const float* g, float eps,
                          void* out, bool out_bf16, hipStream_t s);

// Per-head q/k RMSNorm + split-halves RoPE on q and k, then q -> q_out and k, v -> pool.
struct QkRopeArgs {
  const float* qkv;  // [n_rows][(H + 2 Hkv) D]
  const float* q_norm;
  const float* k_norm;
  const float2* rope;  // [max_context][D/2] (cos, sin)
  void* q_out;         // [n_rows][H][D] in kv dtype
  PoolDev pool;
  int layer;
  int n_heads, n_kv_heads, head_dim;
  float eps;
  bool kv_f16;
  BatchDev b;
};
hipError_t launch_qk_rope_kv(const QkRopeArgs& a, hipStream_t s);
// One (row r, head hh) of the Q|K|V row, its channels j and j + D/2 in lane j < D/2 (x1, x2):
// q and k heads RMS-normalised over D with their gains and rotated by RoPE at the row's
// position, q stored to q_out, k and v to the pool at (table[pos / B], pos % B) (the v head
// as it is). Shared by qk_rope_kv_kernel and the float32 Q|K|V combine, so both give the same
// bits.
template <bool KV_F16>
__device__ __forceinline__ void qk_rope_kv_head(const QkRopeArgs& a, int r, int hh, int lane, float x1, float x2) {
  const int H = a.n_heads, Hkv = a.n_kv_heads, D = a.head_dim, half = D / 2;
  const int pos = a.b.row_pos[r];
  const bool active = lane < half;
  const bool is_v = hh >= H + Hkv;
  if (!is_v) {
    const float2 cs = active ? a.rope[(int64_t)pos * half + lane] : make_float2(1.f, 0.f);
    norm_rope_pair(x1, x2, hh < H ? a.q_norm : a.k_norm, cs, lane, D, a.eps);
  }
  if (!active) return;
  if (hh < H) {
    const int64_t o = ((int64_t)r * H + hh) * D;
    if constexpr (KV_F16) {
      uint16_t* q = (uint16_t*)a.q_out;
      q[o + lane] = f32_to_f16_bits(x1);
      q[o + lane + half] = f32_to_f16_bits(x2);
    } else {
      float* q = (float*)a.q_out;
      q[o + lane] = x1;
      q[o + lane + half] = x2;
    }
    return;
  }
  const int kvh = is_v ? hh - H - Hkv : hh - H;
  const int seq = a.b.row_seq[r];
  const int64_t blk = a.b.block_tables[(int64_t)seq * a.b.tbl_stride + (pos >> a.pool.block_shift)];
  const int64_t off = a.pool.offset(a.layer, is_v ? 1 : 0, blk, kvh, pos & (a.pool.block_tokens - 1));
  if constexpr (KV_F16) {
    uint16_t* p = (uint16_t*)a.pool.base + off;
    p[lane] = f32_to_f16_bits(x1);
    p[lane + half] = f32_to_f16_bits(x2);
  } else {
    float* p = (float*)a.pool.base + off;
    p[lane] = x1;
    p[lane + half] = x2;
  }
}

// Attention of single query rows over their sequence's paged keys, split in
// fixed chunks of keys; writes per-chunk partial (max, sum, unnormalised acc).
struct AttnRowsArgs {
  const void* q;  // [n_rows][H][D] kv dtype
  PoolDev pool;
  int layer;
  int n_heads, n_kv_heads, head_dim;
  bool kv_f16;
  int n_chunks;   // chunks per row in this call (max over rows)
  float* partial; // [n_rows][H][n_chunks][D + 2]
  BatchDev b;
};
int attn_rows_chunk(int head_dim, bool kv_f16, int group);
hipError_t launch_attn_rows(const AttnRowsArgs& a, hipStream_t s);
// The same partials kept in LDS and merged as launch_attn_combine does (identical results), one
// workgroup per (row, KV head), when a.n_chunks <= attn_rows_merged_max_chunks(D, group)
int attn_rows_merged_max_chunks(int head_dim, int group);
hipError_t launch_attn_rows_merged(const AttnRowsArgs& a, void* o, bool out_bf16, hipStream_t s);

// Decode attention: one workgroup per (row, KV head), or per (row, segment, KV head) for rows
// split into segments (a.b.dec_items). It first applies the q/k norm and RoPE of the row
// (qk.qkv) and writes the row's key and value to the pool (segment 0), then attends; chunk
// states merge inside the workgroup. A row of one segment writes o[r][h*D + d] (float32 or
// bf16) directly; a split row's segments write their states to a.partial, laid out
// [rows][H_kv][a.n_chunks slots][group][D + 2] (accumulator, then max and sum; slot n_seg holds
// the new key's state), for launch_attn_decode_combine.
hipError_t launch_attn_decode(const QkRopeArgs& qk, const AttnRowsArgs& a, void* o, bool out_bf16, hipStream_t s);
// The split rows' outputs: their segment states merged in segment order, then the new key's.
hipError_t launch_attn_decode_combine(const AttnRowsArgs& a, void* o, bool out_bf16, hipStream_t s);

// o[r][h*D + d] = combined attention output (float32 or bf16).
hipError_t launch_attn_combine(const float* partial, int n_rows, int n_heads, int head_dim, int n_chunks,
                               int chunk, const int32_t* row_pos, void* o, bool out_bf16, hipStream_t s);

// Flash-style causal prefill attention on an f16 pool (MFMA), query tiles of one sequence
// (BatchDev::tiles lists (sequence, first row) of tiles of kPrefillQueryTile rows).
struct AttnPrefillArgs {
  const uint16_t* q;  // [n_rows][H][D] f16
  PoolDev pool;
  int layer;
  int n_heads, n_kv_heads, head_dim;
  void* o;  // [n_rows][H*D] float32 or bf16
  bool out_bf16;
  BatchDev b;
};
bool attn_prefill_supported(int head_dim, int group);
hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s);

// C[M][N] (epilogue) = A[M][K] . B^T, B = concatenation of weight matrices along N.
enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };
struct GemmArgs {
  const void* A;  // [M][K], float32 (f32 weights) or bf16
  int lda;
  int M, N, K;
  WMat seg[3];  // B segments along N (EPI_SWIGLU: seg[0] gate, seg[1] up, N = ff)
  int nseg;
  void* C;  // float32 [M][ldc] (STORE, RESID) or act dtype (SWIGLU)
  int ldc;
  bool c_bf16;  // SWIGLU output in bf16
  // Decode GEMM only: the RMSNorm in front of a product is deferred, RMSNorm(x) g W =
  // diag(1 / rms(x)) (x g) W. STORE / SWIGLU with ssq_in: A is xg = bf16(x * g), the residual
  // times the norm's gain [M][K] (lda), and each output row is scaled by 1 / sqrt(mean(x^2) +
  // eps), the mean from ssq_in, x's per-row sums of squares in K/16 partials of 16 columns
  // [M][K/16]. RESID: ssq_out receives those partials of the new x [M][N/16], and xg_out (if
  // set) bf16(x_new * gain_next) [M][ldc] for the next product's deferred norm.
  const float* ssq_in;
  float* ssq_out;
  float eps;
  const float* gain_next;
  uint16_t* xg_out;
  // Decode LM head only (optional): per (row, block) greedy candidates, the largest logit of
  // the block's vocabulary share and its lowest id, at [row][block] (see lmhead_decode_parts)
  float* am_v;
  int32_t* am_i;
  // Float32 weights (optional): room for the part sums of products whose grid is split over K
  // (f32_k_parts(epi) * matrices * M * N floats); without it the products take the unsplit kernel
  float* part;
  int64_t part_floats;
  // Float32 residual products split over K (optional, norm_out set): the combine also writes
  // the RMSNorm of each new row of x, x / rms(x) * norm_g with norm_eps, to norm_out (float32
  // [M][N]) with the arithmetic of launch_rmsnorm, so the caller skips that launch; only when
  // gemm_fuses_norm says so
  const float* norm_g;
  float* norm_out;
  float norm_eps;
  // Float32 Q|K|V products split over K (optional, host pointer): the combine applies the q/k
  // norm, RoPE and the K/V write of these arguments (qk_rope_kv_head) to the summed row
  // instead of storing C, so the caller skips launch_qk_rope_kv; only when gemm_fuses_qk says so
  const QkRopeArgs* qk;
};
// Float32 products take K in P fixed parts (part q: steps q * nk / P up to the next), each
// accumulated from zero, the part sums then added in order; P is fixed per epilogue, so per
// product: 16 for the residual products (O, down), 8 for the others
__host__ __device__ constexpr int f32_k_parts(int epi) { return epi == EPI_RESID ? 16 : 8; }
hipError_t launch_gemm(int wdtype, int epi, const GemmArgs& a, hipStream_t s);
// launch_gemm with these arguments also writes the RMSNorm of the new x (norm_out): a float32
// residual product (EPI_RESID) that splits K over blocks, with N one of the vector norm's widths
bool gemm_fuses_norm(int wdtype, int epi, const GemmArgs& a);
// launch_gemm with these arguments does qk's work instead of storing C: a float32 Q|K|V product
// (EPI_STORE, N = (H + 2 H_kv) D, one row per row of qk's batch) that splits K over blocks
bool gemm_fuses_qk(int wdtype, int epi, const GemmArgs& a);

// Prefill GEMM for bf16 / 4-bit weights: 256 x 256 block tiles staged through LDS, the same
// per-element MFMA sequence as launch_gemm (identical results). Epilogues EPI_STORE,
// EPI_RESID, EPI_SWIGLU, and EPI_QKV: the Q|K|V product goes through the per-head q/k
// RMSNorm and RoPE in registers and is stored as q (qk->q_out) and paged K/V (qk->pool), as
// launch_qk_rope_kv does from a stored product.
enum { EPI_QKV = 3 };
bool gemm_big_supported(int wdtype, int epi, int head_dim);
hipError_t launch_gemm_big(int wdtype, int epi, const GemmArgs& a, const QkRopeArgs* qk, hipStream_t s);
// The same kernel on 128 x 128 tiles (bf16 weights; EPI_STORE, EPI_RESID, EPI_SWIGLU), for
// products whose 256 x 256 grid is too small to fill the chip; identical results.
bool gemm_mid_supported(int wdtype, int epi);
hipError_t launch_gemm_mid(int wdtype, int epi, const GemmArgs& a, hipStream_t s);

// The same product for decode steps: K split over up to 8 waves of a block (fixed by K),
// summed in wave order; bf16 and 4-bit weights, K/32 with a supported per-wave step count.
bool gemm_decode_supported(int wdtype, int K);
hipError_t launch_gemm_decode(int wdtype, int epi, const GemmArgs& a, hipStream_t s);

// Decode LM head: logits[M][N] = RMSNorm(x)[M][K] . E^T, taken as xg (a.A = bf16(x * final
// gain), a.lda) . E^T with each row scaled by 1 / rms(x) from a.ssq_in; bf16 / 4-bit E, M <= 64.
bool lmhead_decode_supported(int wdtype, int M, int K);
hipError_t launch_lmhead_decode(int wdtype, const GemmArgs& a, hipStream_t s);
// Blocks of the LM head launch for (M, N): the candidates per row it writes when a.am_v is set,
// or 0 when it writes none for this M (then the logits go through launch_argmax).
int lmhead_decode_parts(int M, int N);

constexpr int kMaxArgmaxParts = 1024;  // greedy candidates per decode row from the LM head, at most

// next[r] = argmax_v logits[r][v], ties to the lowest id; scratch holds argmax_scratch_bytes.
size_t argmax_scratch_bytes(int max_rows, int max_seqs);
hipError_t launch_argmax(const float* logits, int n_rows, int vocab, int32_t* next, void* scratch, hipStream_t s);
// next[r] from nparts candidates per row (values pv[r][j], ids pi[r][j]), same comparison.
hipError_t launch_argmax_final(const float* pv, const int32_t* pi, int n_rows, int nparts, int32_t* next,
                               hipStream_t s);

// Seeded sampling of one token per sequence (dec_sample): sequence s samples row s of logits
// with seqs[s]; counts is the [n_seqs][vocab] count table (zero on entry, left zero).
struct SampleSeq {
  dec_sampling p;
  dec_history h;
};
// vocab <= 262,144
hipError_t launch_sample(const float* logits, int64_t ld, int n_seqs, int vocab, const SampleSeq* seqs,
                         const int32_t* ids, uint32_t* counts, uint64_t* rng, int32_t* next, double* logprob,
                         hipStream_t s);

// Symmetric int4-g32 values q [rows][cols/2] and f16 scales [rows][cols/32] of a float32
// matrix w [rows][cols] (dec_quantize_int4_sym); cols % 32 == 0, 16-byte aligned buffers.
hipError_t launch_quant_int4_sym(const float* w, int64_t rows, int64_t cols, uint8_t* q, uint16_t* scale,
                                 hipStream_t s);

// out[rows][cols] = widened / dequantised matrix (float32).
hipError_t launch_dequant(int wdtype, const WMat& w, int rows, int cols, float* out, hipStream_t s);
// 4-bit matrices (at most kWidenMats, each [rows][cols], cols % 32 == 0) widened to the bf16
// values the 4-bit GEMM kernels stage as MFMA operands, stored row-major at out + out_off[j]
constexpr int kWidenMats = 8;
hipError_t launch_widen_q4(int wdtype, const WMat* mats, const int* cols, const int64_t* out_off, int n,
                           uint16_t* out, hipStream_t s);

}  // namespace dec
