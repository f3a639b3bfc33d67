// Shared definitions of the decoder kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dec.h"

namespace dec {

// ---- vector types ------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- scalar conversions (bit exact, no library rounding modes involved) -------------------

// float -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN (gfx950's
// v_cvt_pk_bf16_f32: one instruction, no per-value branch)
// a 16-byte load at a wave-uniform address plus a 32-bit lane offset, through a raw buffer
// descriptor held in scalar registers (no 64-bit lane addresses). With range 0 the load
// returns zeros without a memory access.
__device__ __forceinline__ u32x4 load_uniform_base(const char* base, uint32_t lane_off, int range = 0x7fffffff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, range, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)lane_off, 0, 0);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values -> packed bf16 pair (lo = a, hi = b), one conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> f16 bits, round to nearest, ties to even (hardware conversion, RNE mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// uint4-g32 weight: (q - zp) * scale as two separately rounded float32 operations.
__device__ __forceinline__ float dequant_u4(uint32_t q, float zp, float scale) {
#pragma clang fp contract(off)
  float t = (float)q - zp;
  return t * scale;
}

// The 4-bit weight formats, groups of 32 input columns. DEC_UINT4_G32: codes u in [0, 15],
// bf16 scale and zero point, w = (u - zp) * scale. DEC_INT4_SYM_G32: two's complement nibbles
// q in [-8, 7] with an f16 scale, w = q * scale ("Candle model runner" 2.5). Flipping a nibble's
// top bit gives u = q + 8, so the signed format is the unsigned one with zp = 8: u - 8 = q is
// exact, and q * scale (at most 15 significant bits) is exact in float32.
constexpr bool is_q4(int wf) { return wf == DEC_UINT4_G32 || wf == DEC_INT4_SYM_G32; }
// packed nibbles (any number per word) as unsigned codes
template <int WF>
__device__ __forceinline__ uint32_t q4_codes(uint32_t packed) {
  return WF == DEC_INT4_SYM_G32 ? packed ^ 0x88888888u : packed;
}
template <int WF>
__device__ __forceinline__ float q4_scale(uint16_t bits) {
  if constexpr (WF == DEC_INT4_SYM_G32)
    return f16_bits_to_f32(bits);
  else
    return bf16_bits_to_f32(bits);
}
// zero point of group gi (the signed format reads none)
template <int WF>
__device__ __forceinline__ float q4_zp(const uint16_t* zp, int64_t gi) {
  if constexpr (WF == DEC_INT4_SYM_G32)
    return 8.0f;
  else
    return bf16_bits_to_f32(zp[gi]);
}

// ---- cross-lane data movement -------------------------------------------------------------
// DPP row operations move data between lanes of a 16-lane row inside a VALU instruction
// (no LDS traffic): quad_perm [1,0,3,2] pairs lanes i ^ 1, quad_perm [2,3,0,1] pairs i ^ 2,
// row_half_mirror pairs i with 7 - i within 8 lanes, row_mirror pairs i with 15 - i.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Sum over aligned groups of WIDTH lanes (WIDTH in 2..64); every lane gets its group's sum.
// Within a 16-lane row the pairing order is fixed, so the result is deterministic.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (WIDTH >= 2) v += dpp<kDppXor1>(v);
  if constexpr (WIDTH >= 4) v += dpp<kDppXor2>(v);
  if constexpr (WIDTH >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (WIDTH >= 16) v += dpp<kDppMirror>(v);
  if constexpr (WIDTH >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (WIDTH >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// SwiGLU of one feature, silu(g) * u = g / (1 + exp(-g)) * u, with the hardware reciprocal
// (within an ulp; the product is rounded to bf16 or kept as float32 after). Every GEMM family
// that can compute a prefill row uses this one expression, so their results stay identical.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---- greedy choice ("Candle model runner" 2.6: greedy takes the argmax, ties to the lowest
// id). Keeps (bv, bi) or takes (v, i) when v is larger, or equal with a lower id; NaN never
// wins. The choice is the same in any order of combination.
__device__ __forceinline__ void greedy_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// ---- wave reductions (fixed butterfly order: deterministic) -------------------------------
template <int WIDTH>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
  return v;
}
// ---- RMSNorm of one row of d = 256 * VPL floats by one wave ("Candle model runner" 2.4:
// x / sqrt(mean(x^2) + eps) * g): lane l holds the row's float4s l + 64 j, j < VPL. Every
// kernel that normalises a row this way calls these, so a row gets the same bits whichever
// kernel computes it (contraction off: no kernel may fuse a square into a sum differently).
template <int VPL>
__device__ __forceinline__ float rms_inv_row(const float4 (&v)[VPL], int d, float eps) {
#pragma clang fp contract(off)
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) ss = ss + (((v[j].x * v[j].x + v[j].y * v[j].y) + v[j].z * v[j].z) + v[j].w * v[j].w);
  ss = wave_sum<64>(ss);
  return 1.0f / sqrtf(ss / (float)d + eps);
}
__device__ __forceinline__ float4 rms_scale4(float4 v, float inv, float4 g) {
#pragma clang fp contract(off)
  return make_float4(v.x * inv * g.x, v.y * inv * g.y, v.z * inv * g.z, v.w * inv * g.w);
}

template <int WIDTH>
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WIDTH));
  return v;
}

// ---- per-head q/k RMSNorm + split-halves RoPE ----------------------------------------------
// Lane j < D/2 holds channels (j, j + D/2) of one head (other lanes hold zeros). RMSNorm over
// the D channels with gain g, then rotation of the pair by the angle's (cos, sin).
// (gains given as the lane's two values g[j], g[j + D/2])
__device__ __forceinline__ void norm_rope_pair_g(float& x1, float& x2, float g1, float g2, float2 cs, int lane, int D,
                                                 float eps) {
  const int half = D / 2;
  const float ss = wave_sum<64>(x1 * x1 + x2 * x2);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  if (lane < half) {
    const float a = x1 * inv * g1;
    const float b = x2 * inv * g2;
    x1 = a * cs.x - b * cs.y;
    x2 = b * cs.x + a * cs.y;
  }
}
__device__ __forceinline__ void norm_rope_pair(float& x1, float& x2, const float* g, float2 cs, int lane, int D,
                                               float eps) {
  const int half = D / 2;
  const float ss = wave_sum<64>(x1 * x1 + x2 * x2);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  if (lane < half) {
    const float a = x1 * inv * g[lane];
    const float b = x2 * inv * g[lane + half];
    x1 = a * cs.x - b * cs.y;
    x2 = b * cs.x + a * cs.y;
  }
}


// ---- per-call batch description (device copies of the host-validated metadata) ------------
struct BatchDev {
  const int32_t* row_tok;      // [n_rows]
  const int32_t* row_pos;      // [n_rows] absolute position
  const int32_t* row_seq;      // [n_rows] sequence index
  const int32_t* seq_start;    // [n_seqs]
  const int32_t* seq_nnew;     // [n_seqs]
  const int32_t* seq_row0;     // [n_seqs] first row of the sequence
  const int32_t* block_tables; // [n_seqs][tbl_stride]
  const int32_t* out_rows;     // [n_out] rows that get logits
  const int32_t* tiles;        // [n_tiles][2] (sequence, first query row) for prefill attention
  // decode attention work items, longest first: [n_dec_items][4] (row, segment, position,
  // sequence), 16-byte aligned; present (n_dec_items > 0) only when some row has more than
  // seg_keys keys before its position, else one item per row in row order is implied
  const int32_t* dec_items;
  int32_t tbl_stride;
  int32_t n_rows, n_seqs, n_out, n_tiles;
  int32_t n_dec_items;
  int32_t seg_keys;            // keys per decode attention segment
};

// Paged KV pool geometry. The pool is [layers][2][n_blocks][Hkv][B][D]; B is a power of two.
struct PoolDev {
  void* base;
  int64_t n_blocks;
  int32_t n_kv_heads, block_tokens, head_dim;
  int32_t block_shift;  // log2(block_tokens)
  __device__ __forceinline__ int64_t slab_elems() const {
    return (int64_t)n_kv_heads * block_tokens * head_dim;
  }
  // element offset of channel 0 of (layer, K=0/V=1, block, kv head, slot)
  __device__ __forceinline__ int64_t offset(int layer, int kv, int64_t block, int h, int slot) const {
    return ((((int64_t)layer * 2 + kv) * n_blocks + block) * n_kv_heads + h) * (int64_t)block_tokens *
               head_dim +
           (int64_t)slot * head_dim;
  }
};

// One weight matrix as a GEMM B operand (rows are output features, [out][in]).
struct WMat {
  const void* w;         // f32 / bf16 values, or 4-bit codes [out][in/2]
  const uint16_t* scale; // 4-bit formats: bf16 (uint4) or f16 (int4 sym) [out][in/32]
  const uint16_t* zp;    // uint4 only
  int32_t rows;
};

}  // namespace dec
