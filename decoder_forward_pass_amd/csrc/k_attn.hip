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
  // keys per lane group per chunk: 32 / GROUP for f16 pools; for float32 pools (16 bytes hold
  // half the channels) 16 / GROUP, so that a chunk's preloaded keys and values fit beside the
  // rest in under 128 registers (four waves per SIMD instead of two)
  static constexpr int KPG = (sizeof(KVT) == 4 ? 16 : 32) / GROUP;
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

template <typename F, int... I>
__device__ __forceinline__ void unrolled_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unrolled(F&& f) {  // f(0), ..., f(N - 1) with constant indices
  unrolled_impl(f, std::make_integer_sequence<int, N>{});
}

// v op v[lane ^ O] for every lane, with no lane-address registers: for O = 16 and 32 the gfx950
// row swaps hand each lane the pair {v[lane], v[lane ^ O]}, for smaller O a bit-mask swizzle
// fetches the partner (op is commutative, so either order gives the same bits)
template <int O, typename Op>
__device__ __forceinline__ float xor_combine(float v, Op op) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    static_assert(O >= 1 && O < 16, "lane distance");
    return op(v, __uint_as_float(__builtin_amdgcn_ds_swizzle((int)u, 0x1F | (O << 10))));
  }
}
template <int FROM, typename Op>
__device__ __forceinline__ float xor_reduce(float v, Op op) {  // over lane bits FROM..32
  if constexpr (FROM < 64) return xor_reduce<FROM * 2>(xor_combine<FROM>(v, op), op);
  return v;
}

// The partial (max, sum, unnormalised accumulator) of one chunk of keys of (row, KV head) for
// its GROUP query heads; lanes of group 0 write head i's D + 2 values through dst(i).
template <typename KVT, int D, int GROUP, typename Dst>
__device__ __forceinline__ void rows_chunk(const AttnRowsArgs& a, int row, int kvh, int chunk, int lane, Dst dst) {
  using G = RowsGeom<KVT, D, GROUP>;
  constexpr int EPL = G::EPL, LPK = G::LPK, KPI = G::KPI, KPG = G::KPG, CHUNK = G::CHUNK;
  const int grp = lane / LPK;
  const int sub = lane % LPK;
  const int Hkv = a.n_kv_heads, H = a.n_heads;
  (void)Hkv;
  const int pos = a.b.row_pos[row];
  const int ctx = pos + 1;
  const int key0 = chunk * CHUNK;
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

  // The KPI keys of one load share a pool block (B is a multiple of KPI), so its id is one
  // scalar load. When the chunk's K and V rows fit in 128 registers of the lane (PRE), all are
  // requested before the scores; otherwise each K row is loaded for its scores and each V row
  // in the second pass.
  constexpr bool PRE = KPG * EPL <= 64;
  auto block_of = [&](int kk) -> int64_t { return table[__builtin_amdgcn_readfirstlane((key0 + kk * KPI) / B)]; };
  auto load_row = [&](int kv_sel, int kk, float (&dst)[EPL]) __attribute__((always_inline)) {
    const int key = key0 + kk * KPI + grp;
    if (key < ctx) {
      load_kv<KVT, EPL>(pool + a.pool.offset(a.layer, kv_sel, block_of(kk), kvh, key % B) + sub * EPL, dst);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) dst[e] = 0.f;
    }
  };
  float kpre[PRE ? KPG : 1][EPL], vpre[PRE ? KPG : 1][EPL];
  if constexpr (PRE) {
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      load_row(0, kk, kpre[kk]);
      load_row(1, kk, vpre[kk]);
    }
  }
  // pass 1: scores of this lane group's keys
  float sc[KPG][GROUP];
#pragma unroll
  for (int kk = 0; kk < KPG; ++kk) {
    const bool valid = key0 + kk * KPI + grp < ctx;
    float kr[EPL];
    if constexpr (PRE) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) kr[e] = kpre[kk][e];
    } else {
      load_row(0, kk, kr);
    }
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d += qv[i][e] * kr[e];
      d = group_sum<LPK>(d);
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
      float v2[EPL];
      if constexpr (PRE) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) v2[e] = vpre[kk][e];
      } else {
        load_row(1, kk, v2);
      }
#pragma unroll
      for (int i = 0; i < GROUP; ++i) {
        const float p = exp2f(sc[kk][i] - m[i]);
        l[i] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[i][e] += p * v2[e];
      }
    }
  }
  const auto add = [](float x, float y) { return x + y; };
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    l[i] = xor_reduce<LPK>(l[i], add);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[i][e] = xor_reduce<LPK>(acc[i][e], add);
  }
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      float* out = dst(i);
#pragma unroll
      for (int e = 0; e < EPL; ++e) out[sub * EPL + e] = acc[i][e];
      if (sub == 0) {
        out[D] = m[i];
        out[D + 1] = l[i];
      }
    }
  }
}

template <typename KVT, int D, int GROUP>
__global__ __launch_bounds__(256) void attn_rows_kernel(AttnRowsArgs a) {
  constexpr int CHUNK = RowsGeom<KVT, D, GROUP>::CHUNK;
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = a.n_chunks;
  const int Hkv = a.n_kv_heads, H = a.n_heads;
  const int chunk = (int)(item % nch);
  const int64_t t = item / nch;
  const int kvh = (int)(t % Hkv);
  const int row = (int)(t / Hkv);
  if (row >= a.b.n_rows) return;
  if (chunk * CHUNK >= a.b.row_pos[row] + 1) return;
  rows_chunk<KVT, D, GROUP>(a, row, kvh, chunk, lane, [&](int i) {
    return a.partial + (((int64_t)row * H + kvh * GROUP + i) * nch + chunk) * (D + 2);
  });
}

// log-sum-exp merge of a row's chunk partials (chunk c at p0 + c * stride: D values, max,
// sum), chunks in ascending order, into the output row of one query head; one wave, lanes over
// the channels
template <bool BF16_OUT>
__device__ __forceinline__ void merge_chunks(const float* p0, int nc, int stride, int D, int lane, void* o,
                                             int64_t ob) {
  float M = -__builtin_inff();
  for (int c = 0; c < nc; ++c) M = fmaxf(M, p0[c * stride + D]);
  float L = 0.f, a0 = 0.f, a1 = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float* p = p0 + c * stride;
    const float sc = exp2f(p[D] - M);
    L += sc * p[D + 1];
    if (lane < D) a0 += sc * p[lane];
    if (lane + 64 < D) a1 += sc * p[lane + 64];
  }
  const float inv = 1.0f / L;
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

// Rows of at most kRowsMergedBytes / (GROUP (D + 2) 4) chunks: one workgroup per (row, KV head);
// its four waves take the chunks in turn, the partials stay in LDS, and the workgroup merges
// them as attn_combine_kernel does (the same arithmetic, so the same results), with no second
// launch.
constexpr int kRowsMergedBytes = 64 * 1024;

template <typename KVT, int D, int GROUP, bool BF16_OUT>
__global__ __launch_bounds__(256) void attn_rows_merged_kernel(AttnRowsArgs a, void* o) {
  constexpr int CHUNK = RowsGeom<KVT, D, GROUP>::CHUNK;
  extern __shared__ __attribute__((aligned(16))) float s_part[];  // [chunk][head][D + 2]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Hkv = a.n_kv_heads, H = a.n_heads;
  const int kvh = blockIdx.x % Hkv, row = blockIdx.x / Hkv;
  const int nc = (a.b.row_pos[row] + CHUNK) / CHUNK;  // chunks holding keys 0..pos
  for (int c = wave; c < nc; c += 4)
    rows_chunk<KVT, D, GROUP>(a, row, kvh, c, lane, [&](int i) { return s_part + ((int64_t)c * GROUP + i) * (D + 2); });
  __syncthreads();
  for (int i = wave; i < GROUP; i += 4)
    merge_chunks<BF16_OUT>(s_part + i * (D + 2), nc, GROUP * (D + 2), D, lane, o,
                           (int64_t)row * H * D + (int64_t)(kvh * GROUP + i) * D);
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

int attn_rows_merged_max_chunks(int head_dim, int group) {
  return kRowsMergedBytes / (group * (head_dim + 2) * 4);
}

template <typename KVT, int D, int GROUP>
static void rows_merged_go(const AttnRowsArgs& a, void* o, bool bf16_out, hipStream_t s) {
  const dim3 g((unsigned)(a.b.n_rows * a.n_kv_heads));
  const uint32_t lds = (uint32_t)(a.n_chunks * GROUP * (D + 2) * 4);
  if (bf16_out)
    launch_kernel(attn_rows_merged_kernel<KVT, D, GROUP, true>, g, dim3(256), lds, s, a, o);
  else
    launch_kernel(attn_rows_merged_kernel<KVT, D, GROUP, false>, g, dim3(256), lds, s, a, o);
}

template <typename KVT, int D>
static hipError_t rows_merged_group(const AttnRowsArgs& a, void* o, bool bf16_out, hipStream_t s) {
  switch (a.n_heads / a.n_kv_heads) {
    case 1: rows_merged_go<KVT, D, 1>(a, o, bf16_out, s); break;
    case 2: rows_merged_go<KVT, D, 2>(a, o, bf16_out, s); break;
    case 4: rows_merged_go<KVT, D, 4>(a, o, bf16_out, s); break;
    case 8: rows_merged_go<KVT, D, 8>(a, o, bf16_out, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_rows_merged(const AttnRowsArgs& a, void* o, bool out_bf16, hipStream_t s) {
  if (a.b.n_rows <= 0) return hipSuccess;
  if (a.n_chunks > attn_rows_merged_max_chunks(a.head_dim, a.n_heads / a.n_kv_heads)) return hipErrorInvalidValue;
  if (a.kv_f16) {
    if (a.head_dim == 32) return rows_merged_group<uint16_t, 32>(a, o, out_bf16, s);
    if (a.head_dim == 64) return rows_merged_group<uint16_t, 64>(a, o, out_bf16, s);
    if (a.head_dim == 128) return rows_merged_group<uint16_t, 128>(a, o, out_bf16, s);
  } else {
    if (a.head_dim == 32) return rows_merged_group<float, 32>(a, o, out_bf16, s);
    if (a.head_dim == 64) return rows_merged_group<float, 64>(a, o, out_bf16, s);
    if (a.head_dim == 128) return rows_merged_group<float, 128>(a, o, out_bf16, s);
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
  merge_chunks<BF16_OUT>(partial + w * nch * (D + 2), nc, D + 2, D, lane, o, (int64_t)row * H * D + (int64_t)h * D);
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

// ---- decode attention: one workgroup per (sequence, KV head) ------------------------------
// A decode step has one query row per sequence. The workgroup's NWV waves take fixed chunks
// of the keys before the new position: wave w handles chunks w, w+NWV, ... in increasing
// order, keeping a running (max, sum, accumulator) per query head. A chunk is two wave-wide
// loads of KPI keys (16 bytes per lane) for K and the same for V; NBUF chunks per wave are in
// flight, in register sets used in turn. The prologue waves first add up the new row's Q|K|V
// partial products, normalise and rotate q and k, and write the new key and value to the pool
// and to LDS; meanwhile every wave has requested its first chunks, whose block ids come from
// one table load per wave. The sequence's block table is copied to LDS for the later chunks,
// so no request after the barrier waits on a table load. The new key enters as one more state
// (its score, sum 1, the new value) merged after the wave states, in wave order, through LDS;
// no partials leave the workgroup. The split depends only on the row's position, so the result
// does not depend on the other sequences.
// A row with more than seg_keys keys before its position is split into segments of seg_keys
// keys, one workgroup each (the work items, longest first, so that the chip stays evenly busy
// over ragged contexts): each runs the same loop over its segment and writes its merged state
// (max, sum, accumulator) unnormalised; segment 0 also writes the pool and the new key's
// state; the combine kernel merges the segments in order, then the new key.

// LDS block-table entries of a decode attention work item: a row of at most seg_keys keys, or
// one segment of a split row, spans at most seg_keys / B + 1 blocks
constexpr int kDecodeTableCap = 1024;
static_assert(kDecodeSegKeys / 16 + 1 <= kDecodeTableCap, "a work item's blocks fit the LDS table (B >= 16)");

template <typename KVT, int D, int GROUP>
struct DecodeGeom {
  static constexpr int EPL = 16 / (int)sizeof(KVT);
  static constexpr int LPK = D / EPL;
  static constexpr int KPI = 64 / LPK;
  static constexpr int DKPG = 2;                   // loads per chunk
  static constexpr int NBUF = GROUP == 4 ? 2 : 3;  // chunk register sets (chunks in flight)
  static constexpr bool QREG = GROUP <= 2;         // query heads held in registers
  static constexpr int CHUNK = DKPG * KPI;
  // waves per workgroup: 16 of at most 128 registers each, or 8 of 256 when eight query heads'
  // accumulators would not fit in 128
  static constexpr int NWV = GROUP >= 8 ? 8 : 16;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
// (taken by value: a bit cast applied directly to an element of an ext_vector is miscompiled
// here into a cast of element 0)
__device__ __forceinline__ half2v as_half2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

template <typename KVT, int D, int GROUP, bool BF16_OUT>
__global__ __launch_bounds__((64 * DecodeGeom<KVT, D, GROUP>::NWV)) void attn_decode_kernel(QkRopeArgs qk,
                                                                                            AttnRowsArgs a, void* out) {
  using G = DecodeGeom<KVT, D, GROUP>;
  constexpr int EPL = G::EPL, LPK = G::LPK, KPI = G::KPI, KPG = G::DKPG, CHUNK = G::CHUNK, NWV = G::NWV;
  constexpr bool F16 = sizeof(KVT) == 2;
  static_assert(CHUNK <= 64 * 16, "a chunk spans at most 64 blocks of 16 positions");
  // per-wave states (max, sum, accumulator); state NWV is the new key's
  __shared__ float s_m[NWV + 1][GROUP], s_l[NWV + 1][GROUP];
  __shared__ float s_acc[NWV][GROUP][D];
  __shared__ __attribute__((aligned(16))) KVT s_q[GROUP + 2][D];  // query heads, new key, new value
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar math
  const int grp = lane / LPK, sub = lane % LPK;
  const int Hkv = a.n_kv_heads, H = a.n_heads;
  const int kvh = blockIdx.x % Hkv;
  int row = blockIdx.x / Hkv, seg = 0, pos, seq;
  if (a.b.n_dec_items) {  // (row, segment, position, sequence) in one load
    const int4 item = ((const int4*)a.b.dec_items)[row];
    row = item.x;
    seg = item.y;
    pos = item.z;
    seq = item.w;
  } else {
    pos = a.b.row_pos[row];
    seq = a.b.row_seq[row];
  }
  // the pool loop covers the keys before the new position (of the segment: keys key_lo ..
  // key_hi - 1); the new key joins at the merge
  const int sk = a.b.seg_keys;
  const int nseg = sk > 0 && pos > sk ? (pos + sk - 1) / sk : 1;
  const int key_lo = seg * sk, key_hi = nseg > 1 ? min(key_lo + sk, pos) : pos;
  const int nch = (key_hi - key_lo + CHUNK - 1) / CHUNK;
  const int32_t* table = a.b.block_tables + (int64_t)seq * a.b.tbl_stride;
  const int bsh = a.pool.block_shift, bmask = a.pool.block_tokens - 1;
  const int first_blk = key_lo >> bsh;  // (segments start at a block boundary)
  const int last_blk = max(key_hi - 1, key_lo) >> bsh;
  const int64_t slab = (int64_t)Hkv * a.pool.block_tokens * D;
  // pool addresses: a wave-uniform part (layer, K or V, KV head, block, the load's first slot)
  // and a 32-bit lane part (the lane group's key within the load, the lane's channels)
  const char* kbase = (const char*)((const KVT*)a.pool.base + (int64_t)a.layer * 2 * a.pool.n_blocks * slab +
                                    (int64_t)kvh * a.pool.block_tokens * D);
  const char* vbase = kbase + a.pool.n_blocks * slab * (int64_t)sizeof(KVT);
  const uint32_t lane_off = (uint32_t)((grp * D + sub * EPL) * sizeof(KVT));

  // The item's block table entries go to LDS (blocks first_blk .. last_blk: at most
  // seg_keys / B + 1 of them, within TCAP) for the requests after the barrier: range-checked
  // loads, so entries past the last block cost nothing. They are waited for together with tab
  // below (which the first requests need), so no later wait depends on them.
  constexpr int TCAP = kDecodeTableCap, TPASS = TCAP / (64 * NWV);
  static_assert(TPASS >= 1, "one table entry per thread at least");
  __shared__ int32_t s_tbl[TCAP];
  uint32_t tcopy[TPASS];
  {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(table + first_blk), 0, min(last_blk - first_blk + 1, TCAP) * 4,
                                          0x00020000);
#pragma unroll
    for (int p = 0; p < TPASS; ++p)
      tcopy[p] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)((p * 64 * NWV + threadIdx.x) * 4), 0, 0);
  }
  // block ids of the wave's first chunks (the ones requested before the barrier): lane j holds
  // block j % bpc of the wave's chunk j / bpc
  const int bpc = CHUNK > a.pool.block_tokens ? CHUNK >> bsh : 1;  // blocks per chunk (64 / bpc >= NBUF)
  const int tab =
      table[min(((key_lo + min(wave + (lane / bpc) * NWV, max(nch - 1, 0)) * CHUNK) >> bsh) + lane % bpc, last_blk)];
  auto publish_table = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < TPASS; ++p) s_tbl[p * 64 * NWV + threadIdx.x] = (int32_t)tcopy[p];
  };

  const int nmine = wave < nch ? (nch - 1 - wave) / NWV + 1 : 0;  // chunks of this wave
  // Requests of chunk ci's K and V rows; SRC picks where the block ids come from: 0 the lanes
  // of tab (the first chunks), 1 the LDS table. Every call issues the same loads whether or
  // not the wave has chunk ci, so that the count of loads in flight is the same on every path
  // (the wait before each chunk then waits for that chunk alone): past nmine the loads have
  // range 0 at a valid address.
  auto issue = [&](auto src, int ci, u32x4 (&kr)[KPG], u32x4 (&vr)[KPG]) __attribute__((always_inline)) {
    constexpr int SRC = decltype(src)::value;
    const bool live = ci < nmine;  // wave-uniform
    const int key0 = key_lo + (wave + ci * NWV) * CHUNK;
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      // the KPI keys of one load share a block (B is a multiple of KPI); keys from key_hi on
      // read a slot of the last block and are masked below
      const int b = min((key0 + kk * KPI) >> bsh, last_blk);
      int blk;
      if constexpr (SRC == 0)
        blk = __builtin_amdgcn_readlane(tab, ci * bpc + b - (key0 >> bsh));
      else
        blk = __builtin_amdgcn_readfirstlane(s_tbl[min(b - first_blk, TCAP - 1)]);
      const int64_t off = ((int64_t)blk * slab + ((key0 + kk * KPI) & bmask) * D) * (int64_t)sizeof(KVT);
      kr[kk] = load_uniform_base(kbase + (live ? off : 0), lane_off, live ? 0x7fffffff : 0);
      vr[kk] = load_uniform_base(vbase + (live ? off : 0), lane_off, live ? 0x7fffffff : 0);
    }
  };
  using FromTab = std::integral_constant<int, 0>;
  using FromLds = std::integral_constant<int, 1>;

  // The row's Q|K|V product gives GROUP + 2 prologue items: query heads kvh*GROUP + it for it < GROUP, then the key and the
  // value; wave w takes items w, w + NWV, ... . An item's loads are issued ahead of the wave's
  // first pool loads, so that they are not queued behind them; the waves without items
  // request their first NBUF chunks at once.
  const int half = D / 2;
  constexpr int NBUF = G::NBUF, NITEM = GROUP + 2;
  u32x4 kb[NBUF][KPG], vb[NBUF][KPG];
  struct Item {
    float x1, x2;  // the lane's two channels (j, j + D/2) of the item's head
    float2 cs;
    float g1, g2;  // q or k norm gains of the lane's two channels
    int newblk;
  };
  auto item_load = [&](int it, Item& t) __attribute__((always_inline)) {
    t.x1 = t.x2 = 0.f;
    t.cs = make_float2(1.f, 0.f);
    t.g1 = t.g2 = 1.f;
    t.newblk = 0;
    if (lane < half) {
      const int hh = it < GROUP ? kvh * GROUP + it : (it == GROUP ? H + kvh : H + Hkv + kvh);
      const float* src = qk.qkv + (int64_t)row * (H + 2 * Hkv) * D + (int64_t)hh * D;
      t.x1 = src[lane];
      t.x2 = src[lane + half];
      if (it <= GROUP) {
        const float* g = it < GROUP ? qk.q_norm : qk.k_norm;
        t.cs = qk.rope[(int64_t)pos * half + lane];
        t.g1 = g[lane];
        t.g2 = g[lane + half];
      }
      if (it >= GROUP) t.newblk = table[pos >> bsh];
    }
  };
  // the new query heads, key and value: normalised and rotated (q, k), rounded to the pool's
  // format into LDS, and the key and value written to the pool at (table[pos / B], pos % B)
  // for later steps
  auto item_finish = [&](int it, const Item& t) __attribute__((always_inline)) {
    float x1 = lane < half ? t.x1 : 0.f, x2 = lane < half ? t.x2 : 0.f;
    if (it <= GROUP) norm_rope_pair_g(x1, x2, t.g1, t.g2, t.cs, lane, D, qk.eps);
    if (lane < half) {
      KVT* dst = s_q[it];
      KVT* pdst = (KVT*)a.pool.base + a.pool.offset(a.layer, it == GROUP ? 0 : 1, t.newblk, kvh, pos & bmask);
      if constexpr (F16) {
        const uint16_t b1 = f32_to_f16_bits(x1), b2 = f32_to_f16_bits(x2);
        dst[lane] = b1;
        dst[lane + half] = b2;
        if (it >= GROUP && seg == 0) {
          pdst[lane] = b1;
          pdst[lane + half] = b2;
        }
      } else {
        dst[lane] = x1;
        dst[lane + half] = x2;
        if (it >= GROUP && seg == 0) {
          pdst[lane] = x1;
          pdst[lane + half] = x2;
        }
      }
    }
  };
  if (wave < NITEM) {
    {
      Item t;
      item_load(wave, t);
      publish_table();
      issue(FromTab{}, 0, kb[0], vb[0]);
      item_finish(wave, t);
    }
    for (int it = wave + NWV; it < NITEM; it += NWV) {
      Item t;
      item_load(it, t);
      item_finish(it, t);
    }
    // (the other chunks are requested only now: their registers and the prologue's would not
    // fit together)
    unrolled<NBUF - 1>([&](auto b) { issue(FromTab{}, b + 1, kb[b + 1], vb[b + 1]); });
  } else {
    publish_table();
    unrolled<NBUF>([&](auto b) { issue(FromTab{}, b, kb[b], vb[b]); });
  }
  __syncthreads();

  // q . k: f16 pairs through v_dot2_f32_f16 (products exact in the float32 sum), float32
  // pools through FMAs; the score is scaled by log2(e)/sqrt(D) afterwards
  const float qscale = 1.4426950408889634f / sqrtf((float)D);
  auto score = [&](const u32x4& q, const u32x4& k) __attribute__((always_inline)) {
    float d = 0.f;
    if constexpr (F16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) d = __builtin_amdgcn_fdot2(as_half2(q[j]), as_half2(k[j]), d, false);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) d += __uint_as_float(q[j]) * __uint_as_float(k[j]);
    }
    return group_sum<LPK>(d) * qscale;
  };
  // (with eight query heads the registers would not hold them beside the chunks: they are
  // then read from LDS for each chunk)
  u32x4 qraw[G::QREG ? GROUP : 1];
  if constexpr (G::QREG) {
#pragma unroll
    for (int i = 0; i < GROUP; ++i) qraw[i] = *(const u32x4*)(&s_q[i][sub * EPL]);
  }
  float m[GROUP], l[GROUP], acc[GROUP][EPL];
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    m[i] = -__builtin_inff();
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;
  }

  // every chunk of the loop holds at least one key before key_hi, so m is finite after it
  auto step = [&](int ci, u32x4 (&kr)[KPG], u32x4 (&vr)[KPG]) __attribute__((always_inline)) {
    const int key0 = key_lo + (wave + ci * NWV) * CHUNK;
    // (an empty barrier keeps the per-chunk LDS reads of the query heads inside the loop, so the
    // compiler does not hold all of them in registers)
    if constexpr (!G::QREG) asm volatile("" ::: "memory");
    float sc[KPG][GROUP];
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      const bool valid = key0 + kk * KPI + grp < key_hi;
#pragma unroll
      for (int i = 0; i < GROUP; ++i) {
        u32x4 q;
        if constexpr (G::QREG)
          q = qraw[i];
        else
          q = *(const u32x4*)(&s_q[i][sub * EPL]);
        const float d = score(q, kr[kk]);
        sc[kk][i] = valid ? d : -__builtin_inff();
      }
    }
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      float mc = sc[0][i];
#pragma unroll
      for (int kk = 1; kk < KPG; ++kk) mc = fmaxf(mc, sc[kk][i]);
      mc = xor_reduce<LPK>(mc, [](float x, float y) { return fmaxf(x, y); });
      const float mn = fmaxf(m[i], mc);
      const float alpha = fast_exp2(m[i] - mn);  // 0 on the first chunk (m = -inf)
      m[i] = mn;
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] *= alpha;
    }
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      // a masked key's slot holds whatever the block holds: zero it, as p * NaN is NaN
      u32x4 vw = vr[kk];
      if (key0 + kk * KPI + grp >= key_hi) vw = u32x4{0u, 0u, 0u, 0u};
      float vv[EPL];
      load_kv<KVT, EPL>((const KVT*)&vw, vv);
#pragma unroll
      for (int i = 0; i < GROUP; ++i) {
        const float p = fast_exp2(sc[kk][i] - m[i]);
        l[i] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[i][e] += p * vv[e];
      }
    }
  };
  // the register sets in turn: while one chunk is consumed the others are in flight, and a
  // set is refilled with the chunk NBUF further on as soon as it has been consumed
  for (int c0 = 0; c0 < nmine; c0 += NBUF) {
    unrolled<NBUF>([&](auto b) {
      const int ci = c0 + b;
      if (ci < nmine) step(ci, kb[b], vb[b]);
      issue(FromLds{}, ci + NBUF, kb[b], vb[b]);
    });
  }

  // this wave's state: sum the lane groups (each holds distinct keys)
  const auto add = [](float x, float y) { return x + y; };
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    l[i] = xor_reduce<LPK>(l[i], add);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[i][e] = xor_reduce<LPK>(acc[i][e], add);
  }
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][i][sub * EPL + e] = acc[i][e];
      if (sub == 0) {
        s_m[wave][i] = m[i];
        s_l[wave][i] = l[i];
      }
    }
  }
  // the new key's state: its score against each query head (computed as in the loop), sum 1,
  // accumulator the new value
  if (wave == NWV - 1) {
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      const float d = score(*(const u32x4*)(&s_q[i][sub * EPL]), *(const u32x4*)(&s_q[GROUP][sub * EPL]));
      if (lane == 0) {
        s_m[NWV][i] = d;
        s_l[NWV][i] = 1.f;
      }
    }
  }
  __syncthreads();
  const int nw = min(NWV, nch);  // waves that saw at least one chunk
  if (nseg > 1) {
    // a segment of a split row: its wave states merged in wave order (every segment has a
    // key, so wave 0 has a state), written unnormalised; segment 0 adds the new key's state
    float* rec = a.partial + ((int64_t)row * Hkv + kvh) * a.n_chunks * (GROUP * (D + 2));
    for (int t = threadIdx.x; t < GROUP * D; t += 64 * NWV) {
      const int i = t / D, d = t % D;
      float M = s_m[0][i];
      for (int w = 1; w < nw; ++w) M = fmaxf(M, s_m[w][i]);
      float L = 0.f, A = 0.f;
      for (int w = 0; w < nw; ++w) {
        const float sc = fast_exp2(s_m[w][i] - M);
        L += sc * s_l[w][i];
        A += sc * s_acc[w][i][d];
      }
      float* r = rec + (int64_t)seg * (GROUP * (D + 2)) + i * (D + 2);
      r[d] = A;
      if (d == 0) {
        r[D] = M;
        r[D + 1] = L;
      }
      if (seg == 0) {
        float* rn = rec + (int64_t)nseg * (GROUP * (D + 2)) + i * (D + 2);
        if constexpr (F16)
          rn[d] = f16_bits_to_f32(s_q[GROUP + 1][d]);
        else
          rn[d] = s_q[GROUP + 1][d];
        if (d == 0) {
          rn[D] = s_m[NWV][i];
          rn[D + 1] = 1.f;
        }
      }
    }
    return;
  }
  // merge: the wave states in wave order, then the new key's
  for (int t = threadIdx.x; t < GROUP * D; t += 64 * NWV) {
    const int i = t / D, d = t % D;
    float M = s_m[NWV][i];
    for (int w = 0; w < nw; ++w) M = fmaxf(M, s_m[w][i]);
    float L = 0.f, A = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float sc = fast_exp2(s_m[w][i] - M);
      L += sc * s_l[w][i];
      A += sc * s_acc[w][i][d];
    }
    float vnew;
    if constexpr (F16)
      vnew = f16_bits_to_f32(s_q[GROUP + 1][d]);
    else
      vnew = s_q[GROUP + 1][d];
    const float sn = fast_exp2(s_m[NWV][i] - M);
    L += sn;
    A += sn * vnew;
    const float v = A / L;
    const int64_t o = (int64_t)row * H * D + (int64_t)(kvh * GROUP + i) * D + d;
    if constexpr (BF16_OUT)
      ((uint16_t*)out)[o] = f32_to_bf16_bits(v);
    else
      ((float*)out)[o] = v;
  }
}

template <typename KVT, int D, int GROUP>
static void decode_launch(const QkRopeArgs& qk, const AttnRowsArgs& a, void* o, bool bf16_out, hipStream_t s) {
  dim3 g((a.b.n_dec_items ? a.b.n_dec_items : a.b.n_rows) * a.n_kv_heads);
  const dim3 blk(64 * DecodeGeom<KVT, D, GROUP>::NWV);
  if (bf16_out)
    launch_kernel(attn_decode_kernel<KVT, D, GROUP, true>, g, blk, 0, s, qk, a, o);
  else
    launch_kernel(attn_decode_kernel<KVT, D, GROUP, false>, g, blk, 0, s, qk, a, o);
}

template <typename KVT, int D>
static hipError_t decode_dispatch_group(const QkRopeArgs& qk, const AttnRowsArgs& a, void* o, bool bf16_out,
                                        hipStream_t s) {
  switch (a.n_heads / a.n_kv_heads) {
    case 1: decode_launch<KVT, D, 1>(qk, a, o, bf16_out, s); break;
    case 2: decode_launch<KVT, D, 2>(qk, a, o, bf16_out, s); break;
    case 4: decode_launch<KVT, D, 4>(qk, a, o, bf16_out, s); break;
    case 8: decode_launch<KVT, D, 8>(qk, a, o, bf16_out, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const QkRopeArgs& qk, const AttnRowsArgs& a, void* o, bool out_bf16, hipStream_t s) {
  if (a.b.n_rows <= 0) return hipSuccess;
  // every work item must fit the kernel's LDS block table
  if (a.b.seg_keys <= 0 || a.b.seg_keys / a.pool.block_tokens + 1 > kDecodeTableCap) return hipErrorInvalidValue;
  if (a.kv_f16) {
    if (a.head_dim == 32) return decode_dispatch_group<uint16_t, 32>(qk, a, o, out_bf16, s);
    if (a.head_dim == 64) return decode_dispatch_group<uint16_t, 64>(qk, a, o, out_bf16, s);
    if (a.head_dim == 128) return decode_dispatch_group<uint16_t, 128>(qk, a, o, out_bf16, s);
  } else {
    if (a.head_dim == 32) return decode_dispatch_group<float, 32>(qk, a, o, out_bf16, s);
    if (a.head_dim == 64) return decode_dispatch_group<float, 64>(qk, a, o, out_bf16, s);
    if (a.head_dim == 128) return decode_dispatch_group<float, 128>(qk, a, o, out_bf16, s);
  }
  return hipErrorInvalidValue;
}

// ---- combine of split decode rows ------------------------------------------------------------
// One block per (row, KV head); rows of one segment return at once. Thread t takes query head
// t / D of the group and channel t % D: M = the largest state max, then the states' sums and
// accumulators scaled by exp2(m - M), added in slot order (segments 0 .. n_seg - 1, then the
// new key's state), and o = A / L.
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(AttnRowsArgs a, void* out) {
  const int Hkv = a.n_kv_heads, G = a.n_heads / Hkv, D = a.head_dim;
  const int row = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
  const int pos = a.b.row_pos[row], sk = a.b.seg_keys;
  if (!(sk > 0 && pos > sk)) return;
  const int nslot = (pos + sk - 1) / sk + 1;
  const float* rec = a.partial + ((int64_t)row * Hkv + kvh) * a.n_chunks * (G * (D + 2));
  // the first U slots are loaded at once (one memory round trip); longer rows (contexts past
  // (U - 1) segments) take further groups of U
  constexpr int U = 8;
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int i = t / D, d = t % D;
    const float* r = rec + i * (D + 2);
    const int64_t st = (int64_t)G * (D + 2);
    float mv[U], lv[U], av[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      // (slots past the row's last read its last slot, and are then discarded)
      const bool in = j < nslot;
      const float* rj = r + min(j, nslot - 1) * st;
      const float m = rj[D], l = rj[D + 1], x = rj[d];
      mv[j] = in ? m : -__builtin_inff();
      lv[j] = in ? l : 0.f;
      av[j] = in ? x : 0.f;
    }
    float M = mv[0];
#pragma unroll
    for (int j = 1; j < U; ++j) M = fmaxf(M, mv[j]);
    for (int j0 = U; j0 < nslot; j0 += U)
#pragma unroll
      for (int j = 0; j < U; ++j)
        if (j0 + j < nslot) M = fmaxf(M, r[(j0 + j) * st + D]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (j < nslot) {
        const float sc = fast_exp2(mv[j] - M);
        L += sc * lv[j];
        A += sc * av[j];
      }
    }
    for (int j0 = U; j0 < nslot; j0 += U)
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (j0 + j < nslot) {
          const float* rj = r + (j0 + j) * st;
          const float sc = fast_exp2(rj[D] - M);
          L += sc * rj[D + 1];
          A += sc * rj[d];
        }
      }
    const float v = A / L;
    const int64_t o = (int64_t)row * a.n_heads * D + (int64_t)(kvh * G + i) * D + d;
    if constexpr (BF16_OUT)
      ((uint16_t*)out)[o] = f32_to_bf16_bits(v);
    else
      ((float*)out)[o] = v;
  }
}

hipError_t launch_attn_decode_combine(const AttnRowsArgs& a, void* o, bool out_bf16, hipStream_t s) {
  if (a.b.n_rows <= 0 || a.b.n_dec_items <= 0) return hipSuccess;
  const dim3 g(a.b.n_rows * a.n_kv_heads), blk(256);
  if (out_bf16)
    launch_kernel(attn_decode_combine_kernel<true>, g, blk, 0, s, a, o);
  else
    launch_kernel(attn_decode_combine_kernel<false>, g, blk, 0, s, a, o);
  return hipGetLastError();
}

}  // namespace dec
