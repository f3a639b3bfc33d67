// Causal grouped-query attention over the paged KV pool.
//
// o_t = sum_{j <= pos(t)} softmax_j(q_t . k_j / sqrt(D)) v_j over the sequence's own keys
// ("Candle model runner" 2.4, second equation), read in place from the pool blocks the
// sequence's table names (block table[j / B], slot j % B). Query head h reads KV head
// h / (H / H_kv).
//
// attn_rows: one wave per (query row, KV head, chunk of keys). The keys of a row are split
// into fixed chunks whose size depends only on (head_dim, kv dtype, group), so a row's
// result never depends on the other rows of the call. Within a wave, a group of LPK lanes
// holds one key (16 bytes per lane), and the wave covers KPI keys per load; scores are
// computed for the whole chunk first, then one max, then exp2 and the value sum, so no
// running rescale is needed. The partial (max, sum, unnormalised accumulator) of each
// chunk goes to a workspace array and attn_combine merges the chunks in order.
#include "kernels.h"

namespace dec {

template <typename KVT, int D, int GROUP>
struct RowsGeom {
  static constexpr int EPL = 16 / (int)sizeof(KVT);  // elements per lane per load
  static constexpr int LPK = D / EPL;                 // lanes per key
  static constexpr int KPI = 64 / LPK;                // keys per wave-wide load
  static constexpr int KPG = 32 / GROUP;              // keys per lane group per chunk
  static constexpr int CHUNK = KPG * KPI;
};

template <typename KVT, int EPL>
__device__ __forceinline__ void load_kv(const KVT* p, float (&v)[EPL]) {
  if constexpr (sizeof(KVT) == 2) {
    const u32x4 w = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = f16_bits_to_f32((uint16_t)(w[i] & 0xffffu));
      v[2 * i + 1] = f16_bits_to_f32((uint16_t)(w[i] >> 16));
    }
  } else {
    const float4 w = *(const float4*)p;
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
  }
}

template <typename KVT, int D, int GROUP>
__global__ __launch_bounds__(256) void attn_rows_kernel(AttnRowsArgs a) {
  using G = RowsGeom<KVT, D, GROUP>;
  constexpr int EPL = G::EPL, LPK = G::LPK, KPI = G::KPI, KPG = G::KPG, CHUNK = G::CHUNK;
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPK;
  const int sub = lane % LPK;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = a.n_chunks;
  const int Hkv = a.n_kv_heads, H = a.n_heads;
  const int chunk = (int)(item % nch);
  const int64_t t = item / nch;
  const int kvh = (int)(t % Hkv);
  const int row = (int)(t / Hkv);
  if (row >= a.b.n_rows) return;
  const int pos = a.b.row_pos[row];
  const int ctx = pos + 1;
  const int key0 = chunk * CHUNK;
  if (key0 >= ctx) return;
  const int seq = a.b.row_seq[row];
  const int32_t* table = a.b.block_tables + (int64_t)seq * a.b.tbl_stride;
  const int B = a.pool.block_tokens;
  const KVT* pool = (const KVT*)a.pool.base;

  // q of the GROUP query heads of this KV head, pre-scaled by log2(e)/sqrt(D)
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  float qv[GROUP][EPL];
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    const KVT* qp = (const KVT*)a.q + ((int64_t)row * H + kvh * GROUP + i) * D + sub * EPL;
    load_kv<KVT, EPL>(qp, qv[i]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[i][e] *= qscale;
  }

  // pass 1: scores of this lane group's keys
  float sc[KPG][GROUP];
#pragma unroll
  for (int kk = 0; kk < KPG; ++kk) {
    const int key = key0 + kk * KPI + grp;
    const bool valid = key < ctx;
    float kv[EPL];
    if (valid) {
      const int64_t blk = table[key / B];
      load_kv<KVT, EPL>(pool + a.pool.offset(a.layer, 0, blk, kvh, key % B) + sub * EPL, kv);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) kv[e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d += qv[i][e] * kv[e];
      d = wave_sum<LPK>(d);
      sc[kk][i] = valid ? d : -__builtin_inff();
    }
  }
  float m[GROUP];
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    float mm = sc[0][i];
#pragma unroll
    for (int kk = 1; kk < KPG; ++kk) mm = fmaxf(mm, sc[kk][i]);
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1) mm = fmaxf(mm, __shfl_xor(mm, o, 64));
    m[i] = mm;
  }

  // pass 2: exp2 and the value sum
  float l[GROUP];
  float acc[GROUP][EPL];
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < KPG; ++kk) {
    const int key = key0 + kk * KPI + grp;
    if (key < ctx) {
      float vv[EPL];
      const int64_t blk = table[key / B];
      load_kv<KVT, EPL>(pool + a.pool.offset(a.layer, 1, blk, kvh, key % B) + sub * EPL, vv);
#pragma unroll
      for (int i = 0; i < GROUP; ++i) {
        const float p = exp2f(sc[kk][i] - m[i]);
        l[i] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[i][e] += p * vv[e];
      }
    }
  }
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      l[i] += __shfl_xor(l[i], o, 64);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] += __shfl_xor(acc[i][e], o, 64);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      float* dst = a.partial + (((int64_t)row * H + kvh * GROUP + i) * nch + chunk) * (D + 2);
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[sub * EPL + e] = acc[i][e];
      if (sub == 0) {
        dst[D] = m[i];
        dst[D + 1] = l[i];
      }
    }
  }
}

template <typename KVT, int D>
static int chunk_for(int group) {
  switch (group) {
    case 1: return RowsGeom<KVT, D, 1>::CHUNK;
    case 2: return RowsGeom<KVT, D, 2>::CHUNK;
    case 4: return RowsGeom<KVT, D, 4>::CHUNK;
    case 8: return RowsGeom<KVT, D, 8>::CHUNK;
  }
  return 0;
}

int attn_rows_chunk(int head_dim, bool kv_f16, int group) {
  if (kv_f16) {
    if (head_dim == 32) return chunk_for<uint16_t, 32>(group);
    if (head_dim == 64) return chunk_for<uint16_t, 64>(group);
    if (head_dim == 128) return chunk_for<uint16_t, 128>(group);
  } else {
    if (head_dim == 32) return chunk_for<float, 32>(group);
    if (head_dim == 64) return chunk_for<float, 64>(group);
    if (head_dim == 128) return chunk_for<float, 128>(group);
  }
  return 0;
}

template <typename KVT, int D>
static hipError_t rows_dispatch_group(const AttnRowsArgs& a, dim3 g, hipStream_t s) {
  switch (a.n_heads / a.n_kv_heads) {
    case 1: attn_rows_kernel<KVT, D, 1><<<g, 256, 0, s>>>(a); break;
    case 2: attn_rows_kernel<KVT, D, 2><<<g, 256, 0, s>>>(a); break;
    case 4: attn_rows_kernel<KVT, D, 4><<<g, 256, 0, s>>>(a); break;
    case 8: attn_rows_kernel<KVT, D, 8><<<g, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_rows(const AttnRowsArgs& a, hipStream_t s) {
  if (a.b.n_rows <= 0) return hipSuccess;
  const int64_t items = (int64_t)a.b.n_rows * a.n_kv_heads * a.n_chunks;
  dim3 g((unsigned)((items + 3) / 4));
  if (a.kv_f16) {
    if (a.head_dim == 32) return rows_dispatch_group<uint16_t, 32>(a, g, s);
    if (a.head_dim == 64) return rows_dispatch_group<uint16_t, 64>(a, g, s);
    if (a.head_dim == 128) return rows_dispatch_group<uint16_t, 128>(a, g, s);
  } else {
    if (a.head_dim == 32) return rows_dispatch_group<float, 32>(a, g, s);
    if (a.head_dim == 64) return rows_dispatch_group<float, 64>(a, g, s);
    if (a.head_dim == 128) return rows_dispatch_group<float, 128>(a, g, s);
  }
  return hipErrorInvalidValue;
}

// ---- combine: log-sum-exp merge of the chunk partials, chunks in ascending order ----------

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ partial, int n_rows,
                                                           int H, int D, int nch, int chunk,
                                                           const int32_t* __restrict__ row_pos,
                                                           void* __restrict__ o) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)n_rows * H) return;
  const int row = (int)(w / H), h = (int)(w % H);
  const int nc = (row_pos[row] + chunk) / chunk;  // chunks holding keys 0..pos
  const float* base = partial + w * nch * (D + 2);
  float M = -__builtin_inff();
  for (int c = 0; c < nc; ++c) M = fmaxf(M, base[c * (D + 2) + D]);
  float L = 0.f, a0 = 0.f, a1 = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float* p = base + c * (D + 2);
    const float sc = exp2f(p[D] - M);
    L += sc * p[D + 1];
    if (lane < D) a0 += sc * p[lane];
    if (lane + 64 < D) a1 += sc * p[lane + 64];
  }
  const float inv = 1.0f / L;
  const int64_t ob = (int64_t)row * H * D + (int64_t)h * D;
  if constexpr (BF16_OUT) {
    uint16_t* out = (uint16_t*)o + ob;
    if (lane < D) out[lane] = f32_to_bf16_bits(a0 * inv);
    if (lane + 64 < D) out[lane + 64] = f32_to_bf16_bits(a1 * inv);
  } else {
    float* out = (float*)o + ob;
    if (lane < D) out[lane] = a0 * inv;
    if (lane + 64 < D) out[lane + 64] = a1 * inv;
  }
}

hipError_t launch_attn_combine(const float* partial, int n_rows, int n_heads, int head_dim, int n_chunks,
                               int chunk, const int32_t* row_pos, void* o, bool out_bf16, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t waves = (int64_t)n_rows * n_heads;
  dim3 g((unsigned)((waves + 3) / 4));
  if (out_bf16)
    attn_combine_kernel<true><<<g, 256, 0, s>>>(partial, n_rows, n_heads, head_dim, n_chunks, chunk, row_pos, o);
  else
    attn_combine_kernel<false><<<g, 256, 0, s>>>(partial, n_rows, n_heads, head_dim, n_chunks, chunk, row_pos, o);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const AttnPrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace dec
