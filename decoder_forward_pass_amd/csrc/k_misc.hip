// Row-wise kernels of the decoder: embedding gather, RMSNorm, fused per-head
// q/k RMSNorm + split-halves RoPE + paged KV write, greedy argmax, and the
// debug dequantisation. Every kernel handles each row independently, so a
// row's result does not depend on the rest of the batch.
#include <algorithm>

#include "kernels.h"

namespace dec {

// ---- embedding ("Candle model runner" 2.4: the LM head is the embedding matrix itself;
// x = E[id] for each new token) -----------------------------------------------------------

template <int WF>
__device__ __forceinline__ void embed_row(const WMat& E, int t, int d, float* __restrict__ xr);

template <int WF>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tok, int vocab, int d,
                                                    WMat E, float* __restrict__ x, float* __restrict__ ssq,
                                                    uint16_t* __restrict__ xg, const float* __restrict__ g) {
  const int r = blockIdx.x;
  const int t = tok[r];
  float* xr = x + (int64_t)r * d;
  if (t < 0 || t >= vocab) {
    for (int i = threadIdx.x; i < d; i += blockDim.x) xr[i] = __builtin_nanf("");
    if (ssq) {
      for (int i = threadIdx.x; i < d / 16; i += blockDim.x) ssq[(int64_t)r * (d / 16) + i] = __builtin_nanf("");
      for (int i = threadIdx.x; i < d; i += blockDim.x) xg[(int64_t)r * d + i] = 0x7fc0;  // NaN
    }
    return;
  }
  embed_row<WF>(E, t, d, xr);
  if (ssq) {
    __syncthreads();  // the row is in global memory; each thread sums its 16-column groups
    for (int i = threadIdx.x; i < d / 16; i += blockDim.x) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) s += xr[16 * i + j] * xr[16 * i + j];
      ssq[(int64_t)r * (d / 16) + i] = s;
    }
    for (int i = threadIdx.x; i < d; i += blockDim.x) xg[(int64_t)r * d + i] = f32_to_bf16_bits(xr[i] * g[i]);
  }
}

template <int WF>
__device__ __forceinline__ void embed_row(const WMat& E, int t, int d, float* __restrict__ xr) {
  if constexpr (WF == DEC_F32) {
    const float* er = (const float*)E.w + (int64_t)t * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) xr[i] = er[i];
  } else if constexpr (WF == DEC_BF16) {
    const uint16_t* er = (const uint16_t*)E.w + (int64_t)t * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) xr[i] = bf16_bits_to_f32(er[i]);
  } else {
    const uint8_t* er = (const uint8_t*)E.w + (int64_t)t * (d / 2);
    const uint16_t* sr = E.scale + (int64_t)t * (d / 32);
    const int64_t g0 = (int64_t)t * (d / 32);
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
      uint32_t byte = q4_codes<WF>(er[i >> 1]);
      uint32_t q = (i & 1) ? ((byte >> 4) & 15u) : (byte & 15u);
      xr[i] = dequant_u4(q, q4_zp<WF>(E.zp, g0 + (i >> 5)), q4_scale<WF>(sr[i >> 5]));
    }
  }
}

hipError_t launch_embed(const int32_t* tok, int n_rows, int vocab, int d, int wdtype, const WMat& E,
                        float* x, float* ssq, uint16_t* xg, const float* gain, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  if (ssq && (!xg || !gain)) return hipErrorInvalidValue;
  dim3 g(n_rows), b(256);
  if (wdtype == DEC_F32)
    embed_kernel<DEC_F32><<<g, b, 0, s>>>(tok, vocab, d, E, x, ssq, xg, gain);
  else if (wdtype == DEC_BF16)
    embed_kernel<DEC_BF16><<<g, b, 0, s>>>(tok, vocab, d, E, x, ssq, xg, gain);
  else if (wdtype == DEC_UINT4_G32)
    embed_kernel<DEC_UINT4_G32><<<g, b, 0, s>>>(tok, vocab, d, E, x, ssq, xg, gain);
  else if (wdtype == DEC_INT4_SYM_G32)
    embed_kernel<DEC_INT4_SYM_G32><<<g, b, 0, s>>>(tok, vocab, d, E, x, ssq, xg, gain);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---- RMSNorm ("Candle model runner" 2.4, first equation: x / sqrt(mean(x^2) + eps) * w) ---
// One wave per row; lane i holds elements i, i+64, ...; the sum of squares is
// added in a fixed order (per lane, then a butterfly), so it is deterministic.

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x,
                                                      const int32_t* __restrict__ rows, int n, int d,
                                                      const float* __restrict__ g, float eps,
                                                      void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const int src = rows ? rows[r] : r;
  const float* xr = x + (int64_t)src * d;
  float ss = 0.f;
  for (int i = lane; i < d; i += 64) ss += xr[i] * xr[i];
  ss = wave_sum<64>(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  if constexpr (BF16_OUT) {
    uint16_t* o = (uint16_t*)out + (int64_t)r * d;
    for (int i = lane; i < d; i += 64) o[i] = f32_to_bf16_bits(xr[i] * inv * g[i]);
  } else {
    float* o = (float*)out + (int64_t)r * d;
    for (int i = lane; i < d; i += 64) o[i] = xr[i] * inv * g[i];
  }
}

// Widths that are multiples of 256: each lane loads its d/256 float4 of the row at once, the
// sum of squares is added per lane in a fixed order and then by a butterfly (rms_inv_row).
template <bool BF16_OUT, int VPL>
__global__ __launch_bounds__(256) void rmsnorm_vec_kernel(const float* __restrict__ x,
                                                          const int32_t* __restrict__ rows, int n, int d,
                                                          const float* __restrict__ g, float eps,
                                                          void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const int src = rows ? rows[r] : r;
  const float4* xr = (const float4*)(x + (int64_t)src * d);
  const float4* g4 = (const float4*)g;
  float4 v[VPL], gv[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    v[j] = xr[lane + 64 * j];
    gv[j] = g4[lane + 64 * j];
  }
  const float inv = rms_inv_row<VPL>(v, d, eps);
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const float4 y = rms_scale4(v[j], inv, gv[j]);
    const int64_t o = (int64_t)r * d + 4 * (lane + 64 * j);
    if constexpr (BF16_OUT) {
      u32x2 w;
      w[0] = pack_bf16x2(y.x, y.y);
      w[1] = pack_bf16x2(y.z, y.w);
      *(u32x2*)((uint16_t*)out + o) = w;
    } else {
      *(float4*)((float*)out + o) = y;
    }
  }
}

template <bool BF16_OUT>
static bool rmsnorm_vec(const float* x, const int32_t* rows, int n, int d, const float* g, float eps, void* out,
                        hipStream_t s) {
  dim3 grid((n + 3) / 4), b(256);
  switch (d) {
    case 256: rmsnorm_vec_kernel<BF16_OUT, 1><<<grid, b, 0, s>>>(x, rows, n, d, g, eps, out); return true;
    case 512: rmsnorm_vec_kernel<BF16_OUT, 2><<<grid, b, 0, s>>>(x, rows, n, d, g, eps, out); return true;
    case 1024: rmsnorm_vec_kernel<BF16_OUT, 4><<<grid, b, 0, s>>>(x, rows, n, d, g, eps, out); return true;
    case 2048: rmsnorm_vec_kernel<BF16_OUT, 8><<<grid, b, 0, s>>>(x, rows, n, d, g, eps, out); return true;
    case 4096: rmsnorm_vec_kernel<BF16_OUT, 16><<<grid, b, 0, s>>>(x, rows, n, d, g, eps, out); return true;
  }
  return false;
}

hipError_t launch_rmsnorm(const float* x, const int32_t* rows, int n, int d, const float* g, float eps,
                          void* out, bool out_bf16, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (out_bf16 ? rmsnorm_vec<true>(x, rows, n, d, g, eps, out, s) : rmsnorm_vec<false>(x, rows, n, d, g, eps, out, s))
    return hipGetLastError();
  dim3 grid((n + 3) / 4), b(256);
  if (out_bf16)
    rmsnorm_kernel<true><<<grid, b, 0, s>>>(x, rows, n, d, g, eps, out);
  else
    rmsnorm_kernel<false><<<grid, b, 0, s>>>(x, rows, n, d, g, eps, out);
  return hipGetLastError();
}

// ---- q/k RMSNorm + RoPE + KV write --------------------------------------------------------
// "A real model in our own decoder": switch 5, an RMSNorm on each query head and each key head
// before RoPE; "Which channels rotate together": channel j pairs with j + D/2. Angle of pair j
// at position p: p * base^(-2j/D) ("Byte-identical...", rope table section), precomputed on the
// host in double precision. Keys/values go to pool block table[pos / B], slot pos % B
// ("Candle model runner" 2.4 and section 3 "Where a key lands").
// One wave per (row, head) over the H query heads, H_kv key heads and H_kv value heads; lane j
// holds the pair (j, j + D/2).

template <bool KV_F16>
__global__ __launch_bounds__(256) void qk_rope_kv_kernel(QkRopeArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x;
  const int hh = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int H = a.n_heads, Hkv = a.n_kv_heads, D = a.head_dim, half = D / 2;
  if (hh >= H + 2 * Hkv) return;
  const float* src = a.qkv + (int64_t)r * (H + 2 * Hkv) * D + (int64_t)hh * D;
  const bool active = lane < half;
  qk_rope_kv_head<KV_F16>(a, r, hh, lane, active ? src[lane] : 0.f, active ? src[lane + half] : 0.f);
}

hipError_t launch_qk_rope_kv(const QkRopeArgs& a, hipStream_t s) {
  if (a.b.n_rows <= 0) return hipSuccess;
  const int heads = a.n_heads + 2 * a.n_kv_heads;
  dim3 g(a.b.n_rows, (heads + 3) / 4), b(256);
  if (a.kv_f16)
    qk_rope_kv_kernel<true><<<g, b, 0, s>>>(a);
  else
    qk_rope_kv_kernel<false><<<g, b, 0, s>>>(a);
  return hipGetLastError();
}

// ---- greedy argmax ("Candle model runner" 2.6: greedy takes the argmax, ties to the lowest
// id). NaN entries never win. -------------------------------------------------------------


// Two passes: 64 slices of each row in parallel, then the 64 candidates of a row in one wave.
// The comparison (larger value, or equal value and lower id) finds the lowest id of the
// maximum in any order of combination.
constexpr int kArgmaxSlices = 64;

__global__ __launch_bounds__(256) void argmax_slices_kernel(const float* __restrict__ logits, int vocab,
                                                            float* __restrict__ pv, int32_t* __restrict__ pi) {
  const int r = blockIdx.y, sl = blockIdx.x;
  const int len = (vocab + kArgmaxSlices - 1) / kArgmaxSlices;
  const int lo = sl * len, hi = min(vocab, lo + len);
  const float* row = logits + (int64_t)r * vocab;
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) greedy_better(bv, bi, row[i], i);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v = __shfl_xor(bv, o, 64);
    int i = __shfl_xor(bi, o, 64);
    greedy_better(bv, bi, v, i);
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k) greedy_better(bv, bi, sv[k], si[k]);
    pv[r * kArgmaxSlices + sl] = bv;
    pi[r * kArgmaxSlices + sl] = bi;
  }
}

__global__ __launch_bounds__(256) void argmax_final_kernel(const float* __restrict__ pv, const int32_t* __restrict__ pi,
                                                           int n_rows, int nparts, int32_t* __restrict__ next) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  float bv = -__builtin_inff();
  int bi = 0x7fffffff;
  for (int j = lane; j < nparts; j += 64) greedy_better(bv, bi, pv[(int64_t)r * nparts + j], pi[(int64_t)r * nparts + j]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v = __shfl_xor(bv, o, 64);
    int i = __shfl_xor(bi, o, 64);
    greedy_better(bv, bi, v, i);
  }
  if (lane == 0) next[r] = bi == 0x7fffffff ? 0 : bi;
}

// (room for kArgmaxSlices candidates per row of a call, or kMaxArgmaxParts per decode row)
size_t argmax_scratch_bytes(int max_rows, int max_seqs) {
  return std::max((size_t)max_rows * kArgmaxSlices, (size_t)max_seqs * kMaxArgmaxParts) * 8;
}

hipError_t launch_argmax_final(const float* pv, const int32_t* pi, int n_rows, int nparts, int32_t* next,
                               hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  argmax_final_kernel<<<(n_rows + 3) / 4, 256, 0, s>>>(pv, pi, n_rows, nparts, next);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int n_rows, int vocab, int32_t* next, void* scratch, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  float* pv = (float*)scratch;
  int32_t* pi = (int32_t*)(pv + (size_t)n_rows * kArgmaxSlices);
  argmax_slices_kernel<<<dim3(kArgmaxSlices, n_rows), 256, 0, s>>>(logits, vocab, pv, pi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_argmax_final(pv, pi, n_rows, kArgmaxSlices, next, s);
}

// ---- debug dequantisation (same device arithmetic as the GEMM B-tile loader and the
// embedding gather) ---------------------------------------------------------------------------

template <int WF>
__global__ __launch_bounds__(256) void dequant_kernel(WMat w, int rows, int cols, float* __restrict__ out) {
  const int64_t total = (int64_t)rows * cols;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols;
    const int c = (int)(i - r * cols);
    float v;
    if constexpr (WF == DEC_F32) {
      v = ((const float*)w.w)[i];
    } else if constexpr (WF == DEC_BF16) {
      v = bf16_bits_to_f32(((const uint16_t*)w.w)[i]);
    } else {
      uint32_t byte = q4_codes<WF>(((const uint8_t*)w.w)[r * (cols / 2) + (c >> 1)]);
      uint32_t q = (c & 1) ? ((byte >> 4) & 15u) : (byte & 15u);
      const int64_t gi = r * (cols / 32) + (c >> 5);
      v = dequant_u4(q, q4_zp<WF>(w.zp, gi), q4_scale<WF>(w.scale[gi]));
    }
    out[i] = v;
  }
}

// ---- 4-bit weights widened to bf16 (prefill calls of many rows) ----------------------------
// Each value is the operand the 4-bit GEMM kernels stage: dequant_u4 of the code with its group's
// zero point and scale, rounded to bf16 by pack_bf16x2 (columns 2j, 2j + 1 from the low and high
// nibble of byte j). Grid row y takes matrix y; one thread per code word (8 columns), one
// 16-byte store.
struct WidenArgs {
  WMat m[kWidenMats];
  int cols[kWidenMats];
  uint32_t words[kWidenMats];  // rows * cols / 8
  int64_t out_off[kWidenMats];
  uint16_t* out;
};

template <int WF>
__global__ __launch_bounds__(256) void widen_q4_kernel(WidenArgs a) {
  const int j = blockIdx.y;
  const WMat m = a.m[j];
  const uint32_t words = a.words[j], wpr = (uint32_t)a.cols[j] / 8, gpr = wpr / 4;
  uint16_t* const out = a.out + a.out_off[j];
  for (uint32_t wi = blockIdx.x * 256u + threadIdx.x; wi < words; wi += gridDim.x * 256u) {
    const uint32_t r = wi / wpr, c8 = wi - r * wpr;
    const uint32_t codes = q4_codes<WF>(((const uint32_t*)m.w)[wi]);
    const uint32_t gi = r * gpr + (c8 >> 2);
    const float zp = q4_zp<WF>(m.zp, gi);
    const float sc = q4_scale<WF>(m.scale[gi]);
    u32x4 v;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = (codes >> (8 * b)) & 0xffu;
      v[b] = pack_bf16x2(dequant_u4(byte & 15u, zp, sc), dequant_u4(byte >> 4, zp, sc));
    }
    *(u32x4*)(out + (size_t)wi * 8) = v;
  }
}

hipError_t launch_widen_q4(int wdtype, const WMat* mats, const int* cols, const int64_t* out_off, int n,
                           uint16_t* out, hipStream_t s) {
  if (n < 1 || n > kWidenMats) return hipErrorInvalidValue;
  WidenArgs a{};
  uint32_t most = 0;
  for (int j = 0; j < n; ++j) {
    const int64_t words = (int64_t)mats[j].rows * (cols[j] / 8);
    if (cols[j] <= 0 || cols[j] % 32 || mats[j].rows <= 0 || words > 0x7fffffff) return hipErrorInvalidValue;
    a.m[j] = mats[j];
    a.cols[j] = cols[j];
    a.words[j] = (uint32_t)words;
    a.out_off[j] = out_off[j];
    most = std::max(most, (uint32_t)words);
  }
  a.out = out;
  const dim3 grid((unsigned)std::min<uint32_t>((most + 255) / 256, 1024), (unsigned)n);
  if (wdtype == DEC_UINT4_G32)
    widen_q4_kernel<DEC_UINT4_G32><<<grid, 256, 0, s>>>(a);
  else if (wdtype == DEC_INT4_SYM_G32)
    widen_q4_kernel<DEC_INT4_SYM_G32><<<grid, 256, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---- symmetric int4-g32 quantisation ("Candle model runner" 2.5, quantising at load) -------
// One thread per group of 32 columns, float32 throughout: s = f16(max|W| / 7) (the quotient
// rounded to nearest even), q = clamp(rint(W / s), -8, 7) with the stored s; a group whose
// largest magnitude is 0 stores s = 0 and q = 0. Nibbles: column 2b low, 2b + 1 high.
__global__ __launch_bounds__(256) void quant_int4_sym_kernel(const float* __restrict__ w, int64_t rows, int64_t cols,
                                                             uint8_t* __restrict__ q, uint16_t* __restrict__ scale) {
  const int64_t ng = cols / 32, total = rows * ng;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / ng, g = i - r * ng;
    const float4* src = (const float4*)(w + r * cols + g * 32);
    float x[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 v = src[j];
      x[4 * j] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
    const _Float16 sh = (_Float16)(amax / 7.0f);
    const float sv = (float)sh;
    u32x4 words = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      int qv = 0;
      if (sv > 0.f) qv = (int)fminf(fmaxf(__builtin_rintf(x[j] / sv), -8.f), 7.f);
      words[j >> 3] |= (uint32_t)(qv & 15) << (4 * (j & 7));
    }
    *(u32x4*)(q + r * (cols / 2) + g * 16) = words;
    scale[i] = __builtin_bit_cast(uint16_t, sh);
  }
}

hipError_t launch_quant_int4_sym(const float* w, int64_t rows, int64_t cols, uint8_t* q, uint16_t* scale,
                                 hipStream_t s) {
  const int64_t total = rows * (cols / 32);
  if (total <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
  quant_int4_sym_kernel<<<blocks, 256, 0, s>>>(w, rows, cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_dequant(int wdtype, const WMat& w, int rows, int cols, float* out, hipStream_t s) {
  const int64_t total = (int64_t)rows * cols;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (wdtype == DEC_F32)
    dequant_kernel<DEC_F32><<<blocks, 256, 0, s>>>(w, rows, cols, out);
  else if (wdtype == DEC_BF16)
    dequant_kernel<DEC_BF16><<<blocks, 256, 0, s>>>(w, rows, cols, out);
  else if (wdtype == DEC_UINT4_G32)
    dequant_kernel<DEC_UINT4_G32><<<blocks, 256, 0, s>>>(w, rows, cols, out);
  else if (wdtype == DEC_INT4_SYM_G32)
    dequant_kernel<DEC_INT4_SYM_G32><<<blocks, 256, 0, s>>>(w, rows, cols, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dec
