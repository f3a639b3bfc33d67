// Projections as MFMA GEMMs: C = A . W^T with W stored [out][in] ("Candle model runner"
// 2.4: W stored [out, in], y = x W^T). A is the activation (float32 for float32 weights,
// bf16 otherwise); W is float32, bf16, or 4-bit dequantised in registers while the tile is
// staged in LDS: uint4-g32 w = (q - zp) * scale ("Byte-identical...", "The bar we set") or
// symmetric int4-g32 w = q * scale ("Candle model runner" 2.5), rounded to bf16 as the MFMA
// operand.
//
// Batch invariance: every output element is accumulated by one MFMA instruction type per
// weight format (v_mfma_f32_16x16x4_f32 or v_mfma_f32_32x32x16_bf16) over K in ascending
// order: bf16 and 4-bit weights into a single accumulator with no split of K, float32 weights
// in fixed parts of K (16 for the residual products, 8 for the others: set by the product
// alone) whose sums are added in part order. The
// row's result therefore does not depend on M, on the tile a row falls in, or on the other
// rows. (The decode kernels below split K by K alone as well, over the waves of a block.)
//
// Epilogues: store float32 (Q/K/V, logits), add into the float32 residual stream (output
// projection, down projection), SwiGLU silu(gate) * up on two B matrices computed by the same
// block ("Candle model runner" 2.4, silu on the gate only). Float32 products split over K
// finish in a combine kernel, which for the residual products can also write the next RMSNorm
// and for Q|K|V in prefill applies the q/k norm, RoPE and K/V write, each through the device
// code the standalone kernels use.
#include "kernels.h"

#include <algorithm>

namespace dec {

// this wave's direct-to-LDS loads of a stage have landed once at most `later` stages' loads
// (PER each) issued after them are outstanding (later in 0 .. MAXL)
template <int PER, int MAXL>
__device__ __forceinline__ void wait_vm_stages(int later) {
  if constexpr (MAXL > 0) {
    if (later >= MAXL) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER * MAXL) : "memory");
      return;
    }
    wait_vm_stages<PER, MAXL - 1>(later);
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// float32 weights: stages of the direct-to-LDS ring (16 K-columns each)
constexpr int kF32Stages = 3;

// Float32 weights: K is taken in P = f32_k_parts(EPI) fixed parts of its 16-column steps (part
// q: steps q nk / P .. (q + 1) nk / P - 1, set by K and the product alone; P = 16 for the
// residual products, 8 for the others). Each part is accumulated from zero in ascending order
// and the part sums are added in part order, ((p0 + p1) + p2) + ... A block takes the parts in
// turn, or, for grids too small to fill the chip (PART), one
// part (blockIdx.z) whose sums go to a.part for gemm_f32_combine; the results are the same.
template <int WF, int EPI, bool PART>
__global__ __launch_bounds__(256) void gemm_tile64(GemmArgs a) {
  constexpr bool F32 = WF == DEC_F32;
  static_assert(!PART || F32, "K parts over blocks: float32 only");
  constexpr int BM = 64, WAVES = 4, BN = BM;
  constexpr int SUB = 2;  // float32: 16 x 16 MFMA blocks per wave, each way
  constexpr int BK = F32 ? 16 : 64;  // elements of K per LDS tile
  constexpr int RW = F32 ? 17 : 36;  // LDS row stride in 32-bit words (padded)
  constexpr int NB = EPI == EPI_SWIGLU ? 2 : 1;
  __shared__ uint32_t As[F32 ? 1 : BM * RW];
  __shared__ uint32_t Bs[NB][F32 ? 1 : BN * RW];
  // float32: the direct-to-LDS ring (stages of 16 K-columns: 8 of 64 rows or 16 of 32 rows)
  extern __shared__ __attribute__((aligned(16))) uint32_t f32_ring[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = WAVES == 4 ? wave >> 1 : 0, wn = WAVES == 4 ? wave & 1 : 0;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = a.M, K = a.K;

  WMat bm[NB];
  int br0;
  if constexpr (EPI == EPI_SWIGLU) {
    bm[0] = a.seg[0];
    bm[1] = a.seg[1];
    br0 = n0;
  } else {
    int s = 0, base = 0;
    while (s < a.nseg - 1 && n0 >= base + a.seg[s].rows) {
      base += a.seg[s].rows;
      ++s;
    }
    bm[0] = a.seg[s];
    br0 = n0 - base;
  }

  // float32 weights: 2 x 2 blocks of 16 x 16 per wave (v_mfma_f32_16x16x4_f32); bf16 / uint4:
  // one 32 x 32 block per wave (v_mfma_f32_32x32x16_bf16, the full-rate bf16 shape)
  f32x4 acc[NB][SUB][SUB];
  f32x4 sum[NB][SUB][SUB];  // float32: the finished parts' sum
  f32x16 acc32[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int i = 0; i < SUB; ++i)
#pragma unroll
      for (int j = 0; j < SUB; ++j) acc[nb][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 16; ++e) acc32[nb][e] = 0.f;
  }

  if constexpr (F32) {
    // float32: both operands go straight from memory to LDS (direct-to-LDS loads) through a
    // ring of FR stages of 16 K-columns, FR - 1 of them in flight, so the K loop is not one
    // memory round trip per 16 columns. A stage holds BM rows of 64 B per operand; chunk c (4
    // floats) of row r sits at position c ^ ((r / 4) % 4), which keeps the 16-row fragment
    // reads on distinct banks. A load fills 16 rows (1 KB: lane l fills row l / 4, position
    // l % 4); the waves share the BM / 16 loads of each operand. The MFMA sequence is the one
    // below.
    constexpr int LPW = BM / 16 / WAVES;     // 16-row loads per operand per wave
    constexpr int FR = kF32Stages, SROWS = BM * 16;  // stages; floats per operand per stage
    float* const ring = reinterpret_cast<float*>(f32_ring);
    const int nk = K / BK;
    constexpr int KP = f32_k_parts(EPI);
    auto kq = [&](int q) { return q * nk / KP; };  // first step of part q
    // this block's steps tbeg + u, u < n (ring stage u % FR)
    const int tbeg = PART ? kq(blockIdx.z) : 0, n = PART ? kq(blockIdx.z + 1) - tbeg : nk;
    const float* asrc[LPW];
    const float* bsrc[NB][LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int lrow = (wave * LPW + i) * 16 + (lane >> 2), lch = (lane & 3) ^ ((lrow >> 2) & 3);
      asrc[i] = (const float*)a.A + (int64_t)min(m0 + lrow, M - 1) * a.lda + lch * 4;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bsrc[nb][i] = (const float*)bm[nb].w + (int64_t)min(br0 + lrow, bm[nb].rows - 1) * K + lch * 4;
    }
    auto dma = [&](int u) {
      const int col = (tbeg + u) * BK;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        float* st = ring + (u % FR) * (1 + NB) * SROWS + (wave * LPW + i) * 256;
        __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + col),
                                         (void __attribute__((address_space(3)))*)st, 16, 0, 0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          __builtin_amdgcn_global_load_lds((const void*)(bsrc[nb][i] + col),
                                           (void __attribute__((address_space(3)))*)(st + (1 + nb) * SROWS), 16, 0,
                                           0);
      }
    };
    for (int u = 0; u < min(n, FR - 1); ++u) dma(u);
    // a part ends: sum = acc (the first part) or sum + acc, and acc restarts; parts end
    // before the first step of the next one
    int q = 0;
    auto fold = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int bi = 0; bi < SUB; ++bi)
#pragma unroll
          for (int bj = 0; bj < SUB; ++bj) {
            sum[nb][bi][bj] = q == 0 ? acc[nb][bi][bj] : sum[nb][bi][bj] + acc[nb][bi][bj];
            acc[nb][bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
      ++q;
    };
    // (a fragment read: row r, chunk ks, lane's k ks * 4 + lane / 16)
    auto frag = [&](const float* S, int r, int ks) {
      return S[r * 16 + ((ks ^ ((r >> 2) & 3)) << 2) + (lane >> 4)];
    };
    for (int u = 0; u < n; ++u) {
      if constexpr (!PART)
        while (q < KP - 1 && u == kq(q + 1)) fold();  // (empty parts fold a zero sum)
      // stage u has landed for this wave once at most the later issued stages' loads are
      // outstanding; the barrier publishes it and frees stage u - 1 (read in the last step)
      const int later = min(FR - 2, n - 1 - u);
      wait_vm_stages<(1 + NB) * LPW, FR - 2>(later);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (u + FR - 1 < n) dma(u + FR - 1);
      const float* As_ = ring + (u % FR) * (1 + NB) * SROWS;
#pragma unroll
      for (int ks = 0; ks < BK / 4; ++ks) {
        float af[SUB];
#pragma unroll
        for (int bi = 0; bi < SUB; ++bi) af[bi] = frag(As_, wm * 32 + bi * 16 + (lane & 15), ks);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int bj = 0; bj < SUB; ++bj) {
            const float bf = frag(As_ + (1 + nb) * SROWS, wn * 32 + bj * 16 + (lane & 15), ks);
#pragma unroll
            for (int bi = 0; bi < SUB; ++bi)
              acc[nb][bi][bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[bi], bf, acc[nb][bi][bj], 0, 0, 0);
          }
      }
    }
    if constexpr (!PART)
      while (q < KP) fold();  // the last part, and any empty ones after the steps
  } else
  for (int k0 = 0; k0 < K; k0 += BK) {
    // ---- stage A
    {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, c8 = c & 7;
        const int gm = min(m0 + row, M - 1);
        const u32x4 v = *(const u32x4*)((const uint16_t*)a.A + (int64_t)gm * a.lda + k0 + c8 * 8);
        *(u32x4*)(As + row * RW + c8 * 4) = v;
      }
    }
    // ---- stage B (one or two matrices)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int brows = bm[nb].rows;
      if constexpr (WF == DEC_BF16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int c = tid + 256 * i;
          const int row = c >> 3, c8 = c & 7;
          const int gr = min(br0 + row, brows - 1);
          const u32x4 v = *(const u32x4*)((const uint16_t*)bm[nb].w + (int64_t)gr * K + k0 + c8 * 8);
          *(u32x4*)(Bs[nb] + row * RW + c8 * 4) = v;
        }
      } else {
        const int row = tid >> 2, kq = (tid & 3) * 16;
        const int gr = min(br0 + row, brows - 1);
        const u32x2 codes =
            *(const u32x2*)((const uint8_t*)bm[nb].w + (int64_t)gr * (K / 2) + (k0 + kq) / 2);
        const int64_t gi = (int64_t)gr * (K / 32) + (k0 + kq) / 32;
        const float zp = q4_zp<WF>(bm[nb].zp, gi);
        const float sc = q4_scale<WF>(bm[nb].scale[gi]);
        uint32_t* d = Bs[nb] + row * RW + kq / 2;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t byte = (q4_codes<WF>(codes[j >> 2]) >> ((j & 3) * 8)) & 0xffu;
          const float lo = dequant_u4(byte & 15u, zp, sc);
          const float hi = dequant_u4(byte >> 4, zp, sc);
          d[j] = pack_bf16x2(lo, hi);
        }
      }
    }
    __syncthreads();

    // ---- MFMA over the tile, K ascending
    {
      // lane l: row l % 32 of its 32-row block, k = 16 ks + 8 (l / 32) .. +8
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const bf16x8 af =
            __builtin_bit_cast(bf16x8, *(const u32x4*)(As + (wm * 32 + (lane & 31)) * RW + ks * 8 + (lane >> 5) * 4));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 bf = __builtin_bit_cast(
              bf16x8, *(const u32x4*)(Bs[nb] + (wn * 32 + (lane & 31)) * RW + ks * 8 + (lane >> 5) * 4));
          acc32[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc32[nb], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue. 16 x 16 blocks: lane holds column lane % 16, rows 4 (lane / 16) + r.
  // 32 x 32 block: lane holds column lane % 32, rows 8 (i / 4) + 4 (lane / 32) + i % 4.
  if constexpr (PART) {
    // the part's sums, at [part][matrix][M][N] of a.part
    float* const dst = a.part + (int64_t)blockIdx.z * NB * M * a.N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int bi = 0; bi < SUB; ++bi)
#pragma unroll
        for (int bj = 0; bj < SUB; ++bj)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * 32 + bi * 16 + (lane >> 4) * 4 + r, nc = n0 + wn * 32 + bj * 16 + (lane & 15);
            if (m < M && nc < a.N) dst[((int64_t)nb * M + m) * a.N + nc] = acc[nb][bi][bj][r];
          }
    return;
  }
  // the 16 outputs of a lane: (row, column, value, SwiGLU up value); the residual values are
  // all requested before any is updated
  constexpr int NE = 16;
  int om[16], on[16];
  float ov[16], ou[16];
  if constexpr (F32) {
#pragma unroll
    for (int bi = 0; bi < SUB; ++bi)
#pragma unroll
      for (int bj = 0; bj < SUB; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = (bi * SUB + bj) * 4 + r;
          om[e] = m0 + wm * 32 + bi * 16 + (lane >> 4) * 4 + r;
          on[e] = n0 + wn * 32 + bj * 16 + (lane & 15);
          ov[e] = sum[0][bi][bj][r];
          ou[e] = sum[NB - 1][bi][bj][r];
        }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      om[i] = m0 + wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      on[i] = n0 + wn * 32 + (lane & 31);
      ov[i] = acc32[0][i];
      ou[i] = acc32[NB - 1][i];
    }
  }
  float xo[16];
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int e = 0; e < NE; ++e) xo[e] = ((const float*)a.C)[(int64_t)min(om[e], M - 1) * a.ldc + min(on[e], a.N - 1)];
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    if (om[e] >= M || on[e] >= a.N) continue;
    const int64_t o = (int64_t)om[e] * a.ldc + on[e];
    if constexpr (EPI == EPI_STORE) {
      ((float*)a.C)[o] = ov[e];
    } else if constexpr (EPI == EPI_RESID) {
      ((float*)a.C)[o] = xo[e] + ov[e];
    } else {
      const float y = silu_mul(ov[e], ou[e]);
      if (a.c_bf16)
        ((uint16_t*)a.C)[o] = f32_to_bf16_bits(y);
      else
        ((float*)a.C)[o] = y;
    }
  }
}

template <int WF, int EPI, bool PART>
static hipError_t tile64_go(const GemmArgs& a, hipStream_t s) {
  // float32: the stage ring in dynamic LDS (stages x (1 + NB) operands x 64 rows x 64 B)
  constexpr int NB = EPI == EPI_SWIGLU ? 2 : 1;
  const uint32_t lds = WF == DEC_F32 ? kF32Stages * (1 + NB) * 64 * 16 * 4 : 0;
  if (lds) {
    static bool attr = false;  // raise the dynamic LDS limit once per instantiation
    if (!attr) {
      hipError_t e = hipFuncSetAttribute((const void*)gemm_tile64<WF, EPI, PART>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr = true;
    }
  }
  const dim3 g((a.N + 63) / 64, (a.M + 63) / 64, PART ? f32_k_parts(EPI) : 1);
  launch_kernel(gemm_tile64<WF, EPI, PART>, g, dim3(256), lds, s, a);
  return hipGetLastError();
}

// The part sums of gemm_tile64<..., PART> added in part order, then the product's
// epilogue, with the same arithmetic as the tile kernel's own epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_combine(GemmArgs a) {
  constexpr int NB = EPI == EPI_SWIGLU ? 2 : 1;
  const int64_t plane = (int64_t)a.M * a.N, total = plane;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int m = (int)(i / a.N), nc = (int)(i - (int64_t)m * a.N);
    float v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float x = a.part[(int64_t)nb * plane + i];
#pragma unroll
      for (int q = 1; q < f32_k_parts(EPI); ++q) x = x + a.part[((int64_t)q * NB + nb) * plane + i];
      v[nb] = x;
    }
    const int64_t o = (int64_t)m * a.ldc + nc;
    if constexpr (EPI == EPI_STORE) {
      ((float*)a.C)[o] = v[0];
    } else if constexpr (EPI == EPI_RESID) {
      ((float*)a.C)[o] = ((const float*)a.C)[o] + v[0];
    } else {
      const float y = silu_mul(v[0], v[NB - 1]);
      if (a.c_bf16)
        ((uint16_t*)a.C)[o] = f32_to_bf16_bits(y);
      else
        ((float*)a.C)[o] = y;
    }
  }
}

// EPI_RESID with the row's RMSNorm: one wave per row m of N = 256 VPL columns. The new x is
// formed per element exactly as in gemm_f32_combine (parts in order, then old x + sum) and
// normalised as launch_rmsnorm does (rms_inv_row / rms_scale4, the same lane layout).
template <int VPL>
__global__ __launch_bounds__(64) void gemm_f32_combine_norm(GemmArgs a) {
  const int m = blockIdx.x, lane = threadIdx.x;
  const int64_t plane = (int64_t)a.M * a.N;
  float* xr = (float*)a.C + (int64_t)m * a.ldc;
  const float4* g4 = (const float4*)a.norm_g;
  float4 v[VPL], gv[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = 4 * (lane + 64 * j);
    const float* p = a.part + (int64_t)m * a.N + c;
    float4 t = *(const float4*)p;
#pragma unroll
    for (int q = 1; q < f32_k_parts(EPI_RESID); ++q) {
      const float4 u = *(const float4*)(p + q * plane);
      t = make_float4(t.x + u.x, t.y + u.y, t.z + u.z, t.w + u.w);
    }
    const float4 old = *(const float4*)(xr + c);
    v[j] = make_float4(old.x + t.x, old.y + t.y, old.z + t.z, old.w + t.w);
    gv[j] = g4[lane + 64 * j];
    *(float4*)(xr + c) = v[j];
  }
  const float inv = rms_inv_row<VPL>(v, a.N, a.norm_eps);
#pragma unroll
  for (int j = 0; j < VPL; ++j)
    *(float4*)(a.norm_out + (int64_t)m * a.N + 4 * (lane + 64 * j)) = rms_scale4(v[j], inv, gv[j]);
}

// EPI_STORE of the Q|K|V product with its q/k norm, RoPE and K/V write: one wave per (row,
// head), lane j < D/2 summing the parts of channels j and j + D/2 as gemm_f32_combine does,
// then the head's arithmetic of qk_rope_kv_kernel (qk_rope_kv_head); C is not written.
template <bool KV_F16>
__global__ __launch_bounds__(256) void gemm_f32_combine_qk(GemmArgs a, QkRopeArgs qk) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x;
  const int hh = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int H = qk.n_heads, Hkv = qk.n_kv_heads, D = qk.head_dim, half = D / 2;
  if (hh >= H + 2 * Hkv) return;
  const int64_t plane = (int64_t)a.M * a.N;
  float x[2] = {0.f, 0.f};
  if (lane < half) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t i = (int64_t)r * a.N + (int64_t)hh * D + lane + e * half;
      float t = a.part[i];
#pragma unroll
      for (int q = 1; q < f32_k_parts(EPI_STORE); ++q) t = t + a.part[q * plane + i];
      x[e] = t;
    }
  }
  qk_rope_kv_head<KV_F16>(qk, r, hh, lane, x[0], x[1]);
}

// float32 products whose 64 x 64 grid has fewer than 256 tiles split K into its parts over
// blocks when the partial buffer holds them (the same results either way)
static bool f32_splits(int epi, const GemmArgs& a) {
  const int NB = epi == EPI_SWIGLU ? 2 : 1;
  const int64_t tiles = (int64_t)((a.N + 63) / 64) * ((a.M + 63) / 64);
  return tiles < 256 && a.part && (int64_t)f32_k_parts(epi) * NB * a.M * a.N <= a.part_floats;
}

bool gemm_fuses_qk(int wdtype, int epi, const GemmArgs& a) {
  if (wdtype != DEC_F32 || epi != EPI_STORE || !a.qk) return false;
  const QkRopeArgs& q = *a.qk;
  return a.M > 0 && a.M == q.b.n_rows && a.N == (q.n_heads + 2 * q.n_kv_heads) * q.head_dim &&
         q.head_dim <= 128 && f32_splits(epi, a);
}

bool gemm_fuses_norm(int wdtype, int epi, const GemmArgs& a) {
  const int n = a.N;
  return wdtype == DEC_F32 && epi == EPI_RESID && a.norm_out && a.norm_g && a.M > 0 && a.ldc % 4 == 0 &&
         (n == 256 || n == 512 || n == 1024 || n == 2048 || n == 4096) && f32_splits(epi, a);
}

template <int WF, int EPI>
static hipError_t tile64_pick(const GemmArgs& a, hipStream_t s) {
  if constexpr (WF == DEC_F32) {
    if (f32_splits(EPI, a)) {
      hipError_t e = tile64_go<WF, EPI, true>(a, s);
      if (e != hipSuccess) return e;
      if (gemm_fuses_qk(WF, EPI, a)) {
        const dim3 g(a.M, (a.qk->n_heads + 2 * a.qk->n_kv_heads + 3) / 4);
        if (a.qk->kv_f16)
          launch_kernel(gemm_f32_combine_qk<true>, g, dim3(256), 0u, s, a, *a.qk);
        else
          launch_kernel(gemm_f32_combine_qk<false>, g, dim3(256), 0u, s, a, *a.qk);
        return hipGetLastError();
      }
      if (gemm_fuses_norm(WF, EPI, a)) {
        switch (a.N) {
          case 256: launch_kernel(gemm_f32_combine_norm<1>, dim3(a.M), dim3(64), 0u, s, a); break;
          case 512: launch_kernel(gemm_f32_combine_norm<2>, dim3(a.M), dim3(64), 0u, s, a); break;
          case 1024: launch_kernel(gemm_f32_combine_norm<4>, dim3(a.M), dim3(64), 0u, s, a); break;
          case 2048: launch_kernel(gemm_f32_combine_norm<8>, dim3(a.M), dim3(64), 0u, s, a); break;
          default: launch_kernel(gemm_f32_combine_norm<16>, dim3(a.M), dim3(64), 0u, s, a); break;
        }
        return hipGetLastError();
      }
      const int64_t total = (int64_t)a.M * a.N;
      const int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
      launch_kernel(gemm_f32_combine<EPI>, dim3(blocks), dim3(256), 0u, s, a);
      return hipGetLastError();
    }
  }
  return tile64_go<WF, EPI, false>(a, s);
}

template <int WF>
static hipError_t gemm_epi(int epi, const GemmArgs& a, hipStream_t s) {
  if (WF == DEC_F32 && a.K % 16) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE: return tile64_pick<WF, EPI_STORE>(a, s);
    case EPI_RESID: return tile64_pick<WF, EPI_RESID>(a, s);
    case EPI_SWIGLU: return tile64_pick<WF, EPI_SWIGLU>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int wdtype, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (wdtype == DEC_F32) return gemm_epi<DEC_F32>(epi, a, s);
  if (wdtype == DEC_BF16) return gemm_epi<DEC_BF16>(epi, a, s);
  if (wdtype == DEC_UINT4_G32) return gemm_epi<DEC_UINT4_G32>(epi, a, s);
  if (wdtype == DEC_INT4_SYM_G32) return gemm_epi<DEC_INT4_SYM_G32>(epi, a, s);
  return hipErrorInvalidValue;
}



// ---- decode GEMM -----------------------------------------------------------------------------
// Used by decode steps only (M = sequences in the step, small). One block computes 16 output
// columns (and the matching 16 up columns for SwiGLU) for up to 32 rows. The K/32 k-steps are
// split into NW equal ranges of NKS steps (NW = 8, or fewer when K/32 is not a multiple of 8;
// both follow from K alone); wave w accumulates its range in ascending order with
// v_mfma_f32_16x16x32_bf16, and the NW partial tiles are added in wave order through LDS. A
// row's result therefore depends on K and the row only, never on how many sequences share
// the step. Every weight and activation fragment of a wave's range is loaded before the first
// MFMA (a scheduling barrier keeps the compiler from sinking the loads to their uses), so the
// weight stream -- the HBM traffic -- is in flight at once.

namespace {

constexpr int kDecWaves = 8;

template <int WF>
struct BRaw;
template <>
struct BRaw<DEC_BF16> {
  u32x4 w;
};
template <>
struct BRaw<DEC_UINT4_G32> {
  uint32_t codes;
  uint16_t scale, zp;
};
template <>
struct BRaw<DEC_INT4_SYM_G32> {
  uint32_t codes;
  uint16_t scale;
};

template <int WF>
__device__ __forceinline__ BRaw<WF> load_b_raw(const WMat& m, int row, int K, int k) {
  BRaw<WF> r;
  if constexpr (WF == DEC_BF16) {
    r.w = *(const u32x4*)((const uint16_t*)m.w + (int64_t)row * K + k);
  } else {
    r.codes = *(const uint32_t*)((const uint8_t*)m.w + (int64_t)row * (K / 2) + k / 2);
    const int64_t gi = (int64_t)row * (K / 32) + k / 32;
    r.scale = m.scale[gi];
    if constexpr (WF == DEC_UINT4_G32) r.zp = m.zp[gi];
  }
  return r;
}

template <int WF>
__device__ __forceinline__ bf16x8 b_frag(const BRaw<WF>& r) {
  if constexpr (WF == DEC_BF16) {
    return __builtin_bit_cast(bf16x8, r.w);
  } else {
    float zp;
    if constexpr (WF == DEC_UINT4_G32)
      zp = bf16_bits_to_f32(r.zp);
    else
      zp = 8.0f;  // signed nibbles read with their top bit flipped
    const float sc = q4_scale<WF>(r.scale);
    const uint32_t codes = q4_codes<WF>(r.codes);
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (codes >> (8 * j)) & 0xffu;
      w[j] = pack_bf16x2(dequant_u4(byte & 15u, zp, sc), dequant_u4(byte >> 4, zp, sc));
    }
    return __builtin_bit_cast(bf16x8, w);
  }
}

}  // namespace

// LDSA: the block's activation rows are staged in LDS by direct-to-LDS loads instead of being
// loaded into registers by each wave. Those rows are the same for every block (they come from
// L2) and the direct path moves them at several times the rate of vector loads. Row r of the
// staged tile keeps its 16-byte chunk c at position c ^ (r % 16), so the 16 rows of a fragment
// read fall on distinct banks; after the products the same LDS holds the wave partials. The
// K split, the order of the additions and the arithmetic are those of the register path.
template <int WF, int EPI, int MT, int NKS, bool LDSA, int RPB = 16 * MT>
__global__ __launch_bounds__(512) void gemm_decode(GemmArgs a, int nw) {
  static_assert(RPB == 16 * MT || (RPB == 8 && MT == 1 && LDSA), "8-row blocks: one 16-row MFMA tile, staged rows");
  // STORE / SWIGLU: A is xg = bf16(x * gain) and each output row is scaled by 1 / rms(x) (the
  // deferred RMSNorm); RESID reads a bf16 activation and writes the sums of squares of the new
  // residual and its gain-scaled bf16 copy for the next product.
  constexpr bool NORM = EPI != EPI_RESID;
  constexpr int NB = EPI == EPI_SWIGLU ? 2 : 1;
  constexpr int ES = 2;  // bytes per activation element (bf16)
  // bf16 weights of single-matrix products staged in LDS as well (the block's 16 rows, same
  // swizzle), right after the activation rows; gate/up (measured slower staged: 128 KB of LDS
  // per block) and uint4 weights are loaded into registers
  constexpr bool BDMA = LDSA && WF == DEC_BF16 && NB == 1;
  constexpr int RED = kDecWaves * NB * MT * 4 * 64;
  __shared__ float red_s[LDSA ? 1 : RED];
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];  // LDSA: [16 MT][K] staged, then partials
  float* red = LDSA ? (float*)s_dyn : red_s;  // [wave][nb][mt][r][lane]
  __shared__ float s_inv[16 * MT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * RPB;
  const int M = a.M, K = a.K;
  const int mend = min(M, m0 + RPB);  // rows of this block: m0 .. mend - 1
  const int cpr = K * ES / 16;  // 16-byte chunks per activation row

  WMat bm[NB];
  int br0;
  if constexpr (EPI == EPI_SWIGLU) {
    bm[0] = a.seg[0];
    bm[1] = a.seg[1];
    br0 = n0;
  } else {
    int s = 0, base = 0;
    while (s < a.nseg - 1 && n0 >= base + a.seg[s].rows) {
      base += a.seg[s].rows;
      ++s;
    }
    bm[0] = a.seg[s];
    br0 = n0 - base;
  }
  const bool active = wave < nw;
  // RESID: the residual values this thread updates in the epilogue, requested with the
  // operand loads instead of after the reduction
  float xres = 0.f, gnext = 0.f;
  if constexpr (EPI == EPI_RESID) {
    if (threadIdx.x < MT * 256) {
      const int t = threadIdx.x, sl = t % 64;
      const int m = m0 + (t / 256) * 16 + (sl >> 4) * 4 + (t / 64) % 4, ncol = n0 + (sl & 15);
      if (m < mend && ncol < a.N) {
        xres = ((const float*)a.C)[(int64_t)m * a.ldc + ncol];
        if (a.xg_out) gnext = a.gain_next[ncol];
      }
    }
  }
  const int brow = min(br0 + (lane & 15), bm[0].rows - 1);
  const int kl = (lane >> 4) * 8;
  const int k0 = wave * NKS * 32 + kl;
  // 4-bit weights, k-steps in fours (WIDE): lane group g = lane / 16 takes a whole 32-column
  // group of its weight row per four MFMAs (16 bytes of codes and one scale in single loads):
  // in k-step 4 j + v it holds columns 32 (4 j + g) + 8 v .. + 8 of the wave's range, and the
  // activation fragments follow the same order. Each k still enters once, and the order does
  // not depend on M.
  constexpr bool WIDE = is_q4(WF) && NKS % 4 == 0;
  auto kof = [&](int i) {  // first of the 8 columns this lane holds in k-step i
    if constexpr (WIDE)
      return wave * NKS * 32 + 32 * (4 * (i >> 2) + (lane >> 4)) + 8 * (i & 3);
    else
      return k0 + i * 32;
  };
  struct BWide {
    u32x4 codes;
    uint16_t scale, zp;
  };
  BRaw<WF> braw[BDMA || WIDE ? 1 : NB][BDMA || WIDE ? 1 : NKS];
  BWide bwide[WIDE ? NB : 1][WIDE ? NKS / 4 : 1];
  u32x4 araw[LDSA ? 1 : MT][LDSA ? 1 : NKS];
  float4 sraw[NORM ? 4 : 1];
  if (active) {
    if constexpr (WIDE) {
#pragma unroll
      for (int j = 0; j < NKS / 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int grp = wave * NKS + 4 * j + (lane >> 4);
          bwide[nb][j].codes = *(const u32x4*)((const uint8_t*)bm[nb].w + (int64_t)brow * (K / 2) + grp * 16);
          const int64_t gi = (int64_t)brow * (K / 32) + grp;
          bwide[nb][j].scale = bm[nb].scale[gi];
          if constexpr (WF == DEC_UINT4_G32) bwide[nb][j].zp = bm[nb].zp[gi];
        }
    } else if constexpr (!BDMA) {
#pragma unroll
      for (int i = 0; i < NKS; ++i)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) braw[nb][i] = load_b_raw<WF>(bm[nb], brow, K, k0 + i * 32);
    }
    if constexpr (!LDSA) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int arow = min(m0 + mt * 16 + (lane & 15), M - 1);
        const uint16_t* ap = (const uint16_t*)a.A + (int64_t)arow * a.lda;
#pragma unroll
        for (int i = 0; i < NKS; ++i) araw[mt][i] = *(const u32x4*)(ap + kof(i));
      }
    }
  }
  if constexpr (LDSA) {
    // every wave stages 1 KB pieces (64 chunk slots, row-major over the swizzled tile)
    const int nins = RPB * cpr / 64;  // (8-row blocks: MFMA rows 8..15 read unstaged LDS; never stored)
    for (int j = wave; j < nins; j += kDecWaves) {
      const int slot = j * 64 + lane, r = slot / cpr, pc = slot % cpr, c = pc ^ (r & 15);
      const uint8_t* src = (const uint8_t*)a.A + ((int64_t)min(m0 + r, M - 1) * a.lda) * ES + c * 16;
      __builtin_amdgcn_global_load_lds((const void*)src, (void __attribute__((address_space(3)))*)(s_dyn + j * 1024),
                                       16, 0, 0);
    }
    if constexpr (BDMA) {
      // the weight rows br0 .. br0 + 15 of each matrix, at byte offset RPB * cpr * 16
      const int nb_ins = NB * 16 * cpr / 64;
      for (int j = wave; j < nb_ins; j += kDecWaves) {
        const int slot = j * 64 + lane, nb = slot / (16 * cpr), rem = slot % (16 * cpr);
        const int r = rem / cpr, pc = rem % cpr, c = pc ^ (r & 15);
        const WMat& w = nb == 0 ? bm[0] : bm[NB - 1];
        const uint8_t* src = (const uint8_t*)w.w + (int64_t)min(br0 + r, w.rows - 1) * K * 2 + c * 16;
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (void __attribute__((address_space(3)))*)(s_dyn + RPB * cpr * 16 + j * 1024),
                                         16, 0, 0);
      }
    }
  }
  // the rows' sums of squares: 4 threads per row, each adding a quarter of the row's K/16
  // partials in order, then the 4 quarters through a fixed DPP pairing
  const int nq = K / 64;
  const float* sp = nullptr;
  if constexpr (NORM) {
    if (threadIdx.x < 64 * MT) {
      sp = a.ssq_in + (int64_t)min(m0 + (int)(threadIdx.x >> 2), M - 1) * (K / 16) + (threadIdx.x & 3) * nq;
      if (nq == 16)
#pragma unroll
        for (int j = 0; j < 4; ++j) sraw[j] = *(const float4*)(sp + 4 * j);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NORM) {
    if (threadIdx.x < 64 * MT) {
      float s = 0.f;
      if (nq == 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) s += sraw[j].x + sraw[j].y + sraw[j].z + sraw[j].w;
      } else {
        for (int j = 0; j < nq; ++j) s += sp[j];
      }
      s += dpp<kDppXor1>(s);
      s += dpp<kDppXor2>(s);
      if ((threadIdx.x & 3) == 0) s_inv[threadIdx.x >> 2] = 1.0f / sqrtf(s / (float)K + a.eps);
    }
  }
  if constexpr (LDSA) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's staging loads have landed
    __syncthreads();
  } else if constexpr (NORM) {
    __syncthreads();
  }
  // fragment of activation row r (local), 8 values from k, from the staged tile
  auto lds_frag = [&](int r, int k, int h) -> u32x4 {
    const int c = (k * ES) / 16 + h;
    return *(const u32x4*)(s_dyn + ((int64_t)r * cpr + (c ^ (r & 15))) * 16);
  };
  // fragment of weight row n (local) of matrix nb, 8 values from k, from the staged weights
  auto lds_bfrag = [&](int nb, int n, int k) -> u32x4 {
    const int c = k / 8;
    return *(const u32x4*)(s_dyn + RPB * cpr * 16 + ((int64_t)(nb * 16 + n) * cpr + (c ^ (n & 15))) * 16);
  };
  f32x4 acc[NB][MT];
  if (active) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NKS; ++i) {
      bf16x8 bf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (BDMA) {
          bf[nb] = __builtin_bit_cast(bf16x8, lds_bfrag(nb, lane & 15, k0 + i * 32));
        } else if constexpr (WIDE) {
          BRaw<WF> r;
          r.codes = bwide[nb][i >> 2].codes[i & 3];
          r.scale = bwide[nb][i >> 2].scale;
          if constexpr (WF == DEC_UINT4_G32) r.zp = bwide[nb][i >> 2].zp;
          bf[nb] = b_frag<WF>(r);
        } else {
          bf[nb] = b_frag<WF>(braw[BDMA || WIDE ? 0 : nb][BDMA || WIDE ? 0 : i]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 af = __builtin_bit_cast(bf16x8, LDSA ? lds_frag(mt * 16 + (lane & 15), kof(i), 0)
                                                          : araw[LDSA ? 0 : mt][LDSA ? 0 : i]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[nb], acc[nb][mt], 0, 0, 0);
      }
    }
  }
  if constexpr (LDSA) __syncthreads();  // the staged tile is done with; the partials reuse it
  if (active) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(((wave * NB + nb) * MT + mt) * 4 + r) * 64 + lane] = acc[nb][mt][r];
  }
  __syncthreads();

  // sum the wave partials in wave order, then the epilogue; thread t -> (mt, r, source lane);
  // a wave covers one (mt, r) for all 64 source lanes, so the 16 columns of a row are 16
  // consecutive lanes
  for (int t = threadIdx.x; t < MT * 4 * 64; t += 512) {
    const int mt = t / 256, r = (t / 64) % 4, sl = t % 64;
    float v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float s = red[((nb * MT + mt) * 4 + r) * 64 + sl];
      for (int w = 1; w < nw; ++w) s += red[(((w * NB + nb) * MT + mt) * 4 + r) * 64 + sl];
      v[nb] = s;
    }
    const int m = m0 + mt * 16 + (sl >> 4) * 4 + r;
    const int ncol = n0 + (sl & 15);
    const bool in = m < mend && ncol < a.N;
    const int64_t o = (int64_t)m * a.ldc + ncol;
    if constexpr (NORM) {  // the deferred RMSNorm of the row
      const float inv = s_inv[mt * 16 + (sl >> 4) * 4 + r];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) v[nb] *= inv;
    }
    if constexpr (EPI == EPI_STORE) {
      if (in) ((float*)a.C)[o] = v[0];
    } else if constexpr (EPI == EPI_RESID) {
      float xn = 0.f;
      if (in) {
        xn = xres + v[0];  // (each thread runs this loop body at most once: MT * 256 <= 512)
        ((float*)a.C)[o] = xn;
        if (a.xg_out) a.xg_out[o] = f32_to_bf16_bits(xn * gnext);
      }
      if (a.ssq_out) {
        const float sq = group_sum<16>(xn * xn);
        if (m < mend && (sl & 15) == 0) a.ssq_out[(int64_t)m * (a.N / 16) + blockIdx.x] = sq;
      }
    } else {
      if (in) {
        const float y = silu_mul(v[0], v[NB - 1]);
        if (a.c_bf16)
          ((uint16_t*)a.C)[o] = f32_to_bf16_bits(y);
        else
          ((float*)a.C)[o] = y;
      }
    }
  }
}

// ---- decode LM head ---------------------------------------------------------------------------
// logits = RMSNorm(x) . E^T for the decode rows (M <= 64). A fixed grid of blocks of 16 waves:
// each block stages the M rows of xg = bf16(x * final gain) once in LDS and takes each row's
// 1 / rms from its sums of squares (the deferred RMSNorm, applied to the logits), then streams
// its contiguous share of the vocabulary in tiles of 16 rows of E, the waves taking the tiles in
// turn. A wave's tiles form one stream of weight-fragment groups (G k-steps each), the next
// group loaded while the current one feeds the MFMAs, across tile boundaries too. Every logit is
// accumulated over the whole K in ascending order -- the same per-element MFMA sequence for any
// number of rows. E is read once per step.

template <int WF, int MT, bool STG>
__global__ __launch_bounds__(1024) void lmhead_decode(GemmArgs a) {
  // [MT*16][K + 8] bf16 rows of xg; with STG, then the block's logits [MT*16][stage stride]
  extern __shared__ __attribute__((aligned(16))) uint16_t s_h[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = a.M, K = a.K, KS = K + 8;
  const int rows = MT * 16;
  // the rows of xg = bf16(x * final gain) into LDS, and each row's 1 / rms (the deferred
  // RMSNorm): 32 threads per row (a wave half), each 1/32 of the row and of its sums of squares
  __shared__ float s_inv[MT * 16];
  {
    const int per = K / 32, nq = K / 16, qper = (nq + 31) / 32;
    for (int r0 = 0; r0 < rows; r0 += 32) {
      const int r = r0 + (threadIdx.x >> 5);
      const int c0 = (threadIdx.x & 31) * per;
      const bool live = r < rows;
      const uint16_t* xr = (const uint16_t*)a.A + (int64_t)min(r, M - 1) * a.lda + c0;
      const float* sp = a.ssq_in + (int64_t)min(r, M - 1) * nq;
      const int q0 = (threadIdx.x & 31) * qper, q1 = min(nq, q0 + qper);
      float ss = 0.f;
      if (live) {
        for (int j = q0; j < q1; ++j) ss += sp[j];
        for (int j = 0; j < per; j += 8) *(u32x4*)(s_h + r * KS + c0 + j) = *(const u32x4*)(xr + j);
      }
      ss = group_sum<32>(ss);
      if (live && (threadIdx.x & 31) == 0) s_inv[r] = 1.0f / sqrtf(ss / (float)K + a.eps);
    }
  }
  __syncthreads();
  // this block's tiles of 16 vocabulary rows: [t0, t1); wave w takes t0 + w, t0 + w + 16, ...
  const WMat E = a.seg[0];
  const int ntiles = (a.N + 15) / 16;
  const int t0 = (int)((int64_t)ntiles * blockIdx.x / gridDim.x);
  const int t1 = (int)((int64_t)ntiles * (blockIdx.x + 1) / gridDim.x);
  const int mine = t0 + wave < t1 ? (t1 - 1 - t0 - wave) / 16 + 1 : 0;
  constexpr int G = 8;  // k-steps per group of weight loads
  const int ksteps = K / 32, gpt = (ksteps + G - 1) / G, total = mine * gpt;
  const int kl = (lane >> 4) * 8;
  auto load_group = [&](int j, BRaw<WF> (&dst)[G]) {
    const int tile = t0 + wave + (j / gpt) * 16, kg = (j % gpt) * G;
    const int brow = min(tile * 16 + (lane & 15), E.rows - 1);
#pragma unroll
    for (int i = 0; i < G; ++i) dst[i] = load_b_raw<WF>(E, brow, K, min(kg + i, ksteps - 1) * 32 + kl);
  };
  // 4-bit E (WIDE; K % 256 == 0, so groups are whole): lane group g = lane / 16 takes a whole
  // 32-column group of its row per four MFMAs, as in the decode GEMM: in k-step kg + 4 h + v it
  // holds columns 32 (kg + 4 h + g) + 8 v .. + 8, and the activation fragments follow
  constexpr bool WIDE = is_q4(WF);
  struct BWide {
    u32x4 codes;
    uint16_t scale, zp;
  };
  auto load_wide = [&](int j, BWide (&dst)[G / 4]) {
    const int tile = t0 + wave + (j / gpt) * 16, kg = (j % gpt) * G;
    const int brow = min(tile * 16 + (lane & 15), E.rows - 1);
#pragma unroll
    for (int h = 0; h < G / 4; ++h) {
      const int grp = kg + 4 * h + (lane >> 4);
      dst[h].codes = *(const u32x4*)((const uint8_t*)E.w + (int64_t)brow * (K / 2) + grp * 16);
      const int64_t gi = (int64_t)brow * (K / 32) + grp;
      dst[h].scale = E.scale[gi];
      if constexpr (WF == DEC_UINT4_G32) dst[h].zp = E.zp[gi];
    }
  };
  auto kof = [&](int kg, int i) {  // first of the 8 columns this lane holds in k-step kg + i
    if constexpr (WIDE)
      return 32 * (kg + 4 * (i >> 2) + (lane >> 4)) + 8 * (i & 3);
    else
      return (kg + i) * 32 + kl;
  };
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // greedy candidates (a.am_v set, MT <= 2): per lane, the best logit and id of its column over
  // the tiles it computes, for each of its rows
  constexpr bool AMX = MT <= 2;
  const bool amx = AMX && a.am_v != nullptr;
  float bv[AMX ? MT : 1][4];
  int bi[AMX ? MT : 1][4];
#pragma unroll
  for (int mt = 0; mt < (AMX ? MT : 1); ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bv[mt][r] = -__builtin_inff();
      bi[mt][r] = 0x7fffffff;
    }
  if constexpr (!WIDE) {
    // bf16 E: two register sets of G k-steps used in turn; group j + 1 is requested before
    // group j feeds the MFMAs. Every group issues the same memory operations, so that each
    // wait covers exactly what it needs: a group with no tile is requested with an empty range
    // (zeros, no memory access, at a valid address), and the stores of a group have an empty
    // range unless it finishes a tile (or, with STG, a round).
    //
    // STG (the logits of a round fit in LDS): the block works in rounds; in round r wave w
    // takes tile t0 + 16 r + w, so a round covers 256 adjacent columns. Every wave runs every
    // round and the block meets after each: the round's logits gather in LDS, leave as whole
    // 16-byte pieces of each row while the next round streams in, and the greedy candidates are
    // taken from LDS. Without STG each tile's logits leave from registers, as 64-byte pieces
    // of four rows (partial cache lines, which cost several times their bytes).
    const int nrounds = (t1 - t0 + 15) / 16;
    const int ngroups = STG ? nrounds * gpt : total;  // groups each wave runs
    auto tile_of = [&](int j) { return STG ? t0 + 16 * (j / gpt) + wave : t0 + wave + (j / gpt) * 16; };
    auto load = [&](int j, u32x4 (&dst)[G]) __attribute__((always_inline)) {
      const bool live = j < ngroups && tile_of(j) < t1;
      const int tile = live ? tile_of(j) : 0, kg = live ? (j % gpt) * G : 0;
      const char* base = (const char*)E.w + (int64_t)tile * 16 * K * 2;  // the tile's first row
      const uint32_t roff = (uint32_t)((min(tile * 16 + (lane & 15), E.rows - 1) - tile * 16) * K) * 2;
#pragma unroll
      for (int i = 0; i < G; ++i)
        dst[i] = load_uniform_base(base, roff + (uint32_t)(min(kg + i, ksteps - 1) * 32 + kl) * 2,
                                   live ? 0x7fffffff : 0);
    };
    auto consume = [&](int j, const u32x4 (&src)[G]) __attribute__((always_inline)) {
      const int kg = (j % gpt) * G;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        if (kg + i < ksteps) {
          const bf16x8 bf = __builtin_bit_cast(bf16x8, src[i]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const bf16x8 af = __builtin_bit_cast(bf16x8, *(const u32x4*)(s_h + (mt * 16 + (lane & 15)) * KS +
                                                                         kof(kg, i)));
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[mt], 0, 0, 0);
          }
        }
      }
    };
    // STG: the round stage [2][MT * 16][RS] after the activation rows; thread t keeps the
    // greedy best of row t / 32 over columns 8 (t % 32) .. + 7 of every round
    constexpr int RS = 256 + 4;
    float* const rst = (float*)(s_h + MT * 16 * KS);
    const int grow = threadIdx.x >> 5, gcol = (threadIdx.x & 31) * 8;
    float gbv = -__builtin_inff();
    int gbi = 0x7fffffff;
    auto finish = [&](int j) __attribute__((always_inline)) {
      const bool end = j >= 0 && j < ngroups && j % gpt == gpt - 1;  // group j completes a tile
      const int tile = tile_of(max(j, 0));
      const int ncol = tile * 16 + (lane & 15);
      if constexpr (STG) {
        const int r = max(j, 0) / gpt;
        float* const st = rst + (r & 1) * MT * 16 * RS;
        const int rc0 = (t0 + 16 * r) * 16;                 // the round's first column
        const int rcols = max(0, min(256, min(t1 * 16, a.N) - rc0));  // its columns (a multiple of 4)
        if (end) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int m = mt * 16 + (lane >> 4) * 4 + q;
              st[m * RS + wave * 16 + (lane & 15)] = acc[mt][q] * s_inv[m];
            }
            acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          // (the stage writes are done; the loads in flight stay in flight: no fence on them)
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          if (amx && grow < M) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (gcol + e < rcols) greedy_better(gbv, gbi, st[grow * RS + gcol + e], rc0 + gcol + e);
          }
        }
        // the round's rows, 16 bytes a thread per store (an empty range on the other groups)
        const __amdgpu_buffer_rsrc_t cr =
            __builtin_amdgcn_make_buffer_rsrc(a.C, 0, end ? M * a.ldc * 4 : 0, 0x00020000);
#pragma unroll
        for (int q = 0; q < MT * 16 * 64 / 1024; ++q) {
          const int idx = threadIdx.x + 1024 * q, row = idx >> 6, c4 = (idx & 63) * 4;
          const bool in = end && row < M && c4 < rcols;
          const u32x4 v = in ? *(const u32x4*)(st + row * RS + c4) : u32x4{0u, 0u, 0u, 0u};
          __builtin_amdgcn_raw_buffer_store_b128(v, cr, in ? (int)((row * a.ldc + rc0 + c4) * 4) : (int)0x80000000u,
                                                 0, 0);
        }
      } else {
        const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((float*)a.C + (end ? (int64_t)tile * 16 : 0)), 0, end ? ((M - 1) * a.ldc + 16) * 4 : 0,
            0x00020000);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = mt * 16 + (lane >> 4) * 4 + q;
            const float logit = acc[mt][q] * s_inv[m];
            const bool in = m < M && ncol < a.N;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(logit), cr,
                                                  in ? (int)((m * a.ldc + (lane & 15)) * 4) : (int)0x80000000u, 0, 0);
            if constexpr (AMX)
              if (amx && end && in) greedy_better(bv[AMX ? mt : 0][q], bi[AMX ? mt : 0][q], logit, ncol);
          }
          if (end) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    };
    u32x4 ga[G], gb[G];
    load(0, ga);
    // (stores with an empty range after the first loads, as every later group has them: the
    // loop is then entered with the operations in flight that each later pass sees, so its waits
    // are not taken for the first pass's smaller count)
    finish(-1);
    for (int j = 0; j < ngroups; j += 2) {
      load(j + 1, gb);
      consume(j, ga);
      finish(j);
      load(j + 2, ga);
      consume(j + 1, gb);  // (past the last group: zeros into a cleared accumulator)
      finish(j + 1);
    }
    if constexpr (STG) {
      // the greedy candidates: the 32 threads of a row (half a wave) in a fixed butterfly
      if (amx) {
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
          const float v = __shfl_xor(gbv, o, 64);
          const int i = __shfl_xor(gbi, o, 64);
          greedy_better(gbv, gbi, v, i);
        }
        if ((threadIdx.x & 31) == 0 && grow < M) {
          a.am_v[(int64_t)grow * gridDim.x + blockIdx.x] = gbv;
          a.am_i[(int64_t)grow * gridDim.x + blockIdx.x] = gbi;
        }
      }
      return;
    }
  } else {
  BRaw<WF> cur[WIDE ? 1 : G], nxt[WIDE ? 1 : G];
    BWide wcur[WIDE ? G / 4 : 1], wnxt[WIDE ? G / 4 : 1];
    if (total > 0) {
      if constexpr (WIDE)
        load_wide(0, wcur);
      else
        load_group(0, cur);
    }
    for (int j = 0; j < total; ++j) {
      if (j + 1 < total) {
        if constexpr (WIDE)
          load_wide(j + 1, wnxt);
        else
          load_group(j + 1, nxt);
      }
      const int kg = (j % gpt) * G;
  #pragma unroll
      for (int i = 0; i < G; ++i) {
        if (kg + i < ksteps) {
          bf16x8 bf;
          if constexpr (WIDE) {
            BRaw<WF> r;
            r.codes = wcur[i >> 2].codes[i & 3];
            r.scale = wcur[i >> 2].scale;
            if constexpr (WF == DEC_UINT4_G32) r.zp = wcur[i >> 2].zp;
            bf = b_frag<WF>(r);
          } else {
            bf = b_frag<WF>(cur[WIDE ? 0 : i]);
          }
  #pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const bf16x8 af = __builtin_bit_cast(bf16x8, *(const u32x4*)(s_h + (mt * 16 + (lane & 15)) * KS +
                                                                         kof(kg, i)));
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[mt], 0, 0, 0);
          }
        }
      }
      if (j % gpt == gpt - 1) {  // the tile is complete: store its logits, start the next one
        const int tile = t0 + wave + (j / gpt) * 16;
        const int ncol = tile * 16 + (lane & 15);
  #pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = mt * 16 + (lane >> 4) * 4 + r;
            const float logit = acc[mt][r] * s_inv[m];
            if (m < M && ncol < a.N) {
              ((float*)a.C)[(int64_t)m * a.ldc + ncol] = logit;
              if constexpr (AMX)
                if (amx) greedy_better(bv[AMX ? mt : 0][r], bi[AMX ? mt : 0][r], logit, ncol);
            }
          }
          acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if constexpr (WIDE) {
  #pragma unroll
        for (int h = 0; h < G / 4; ++h) wcur[h] = wnxt[h];
      } else {
  #pragma unroll
        for (int i = 0; i < G; ++i) cur[i] = nxt[i];
      }
    }
  }
  if constexpr (AMX) {
    if (amx) {
      // the 16 lanes of a row group (distinct columns), then the 16 waves through LDS, then one
      // candidate per (row, block)
      __shared__ float s_bv[16][MT * 16];
      __shared__ int s_bi[16][MT * 16];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            const float v = __shfl_xor(bv[mt][r], o, 64);
            const int i = __shfl_xor(bi[mt][r], o, 64);
            greedy_better(bv[mt][r], bi[mt][r], v, i);
          }
          if ((lane & 15) == 0) {
            s_bv[wave][mt * 16 + (lane >> 4) * 4 + r] = bv[mt][r];
            s_bi[wave][mt * 16 + (lane >> 4) * 4 + r] = bi[mt][r];
          }
        }
      __syncthreads();
      const int m = threadIdx.x;
      if (m < MT * 16 && m < M) {
        float v = s_bv[0][m];
        int i = s_bi[0][m];
        for (int w = 1; w < 16; ++w) greedy_better(v, i, s_bv[w][m], s_bi[w][m]);
        a.am_v[(int64_t)m * gridDim.x + blockIdx.x] = v;
        a.am_i[(int64_t)m * gridDim.x + blockIdx.x] = i;
      }
    }
  }
}

// dynamic LDS of the decode LM head at most: a compute unit's 160 KB (gfx950) less 8 KB for the
// kernel's static arrays (s_inv and the greedy candidates, 4.2 KB at 64 rows)
constexpr size_t kLmheadLdsMax = (160 - 8) * 1024;

// one block per compute unit, or fewer when the vocabulary is small
static int lmhead_blocks(int N) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return std::max(1, std::min(std::min(cus, kMaxArgmaxParts), (N + 255) / 256));
}

int lmhead_decode_parts(int M, int N) { return M >= 1 && M <= 32 ? lmhead_blocks(N) : 0; }

template <int WF, int MT, bool STG>
static hipError_t lmhead_go_stg(const GemmArgs& a, size_t lds, int blocks, hipStream_t s) {
  static bool attr = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)lmhead_decode<WF, MT, STG>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLmheadLdsMax);
    if (e != hipSuccess) return e;
    attr = true;
  }
  launch_kernel(lmhead_decode<WF, MT, STG>, dim3(blocks), dim3(1024), (uint32_t)lds, s, a);
  return hipGetLastError();
}

template <int WF, int MT>
static hipError_t lmhead_go(const GemmArgs& a, hipStream_t s) {
  const int blocks = lmhead_blocks(a.N);
  const size_t lds = (size_t)MT * 16 * (a.K + 8) * 2;
  const size_t stage = (size_t)2 * MT * 16 * (256 + 4) * 4;  // two rounds of logits
  if (WF == DEC_BF16 && MT <= 2 && a.N % 4 == 0 && a.ldc % 4 == 0 && lds + stage <= kLmheadLdsMax)
    return lmhead_go_stg<WF, MT, true>(a, lds + stage, blocks, s);
  return lmhead_go_stg<WF, MT, false>(a, lds, blocks, s);
}

bool lmhead_decode_supported(int wdtype, int M, int K) {
  // each of 32 threads per row stages K/32 columns in 16-byte steps
  return (wdtype == DEC_BF16 || is_q4(wdtype)) && M <= 64 && K % 256 == 0 && (size_t)64 * (K + 8) * 2 <= 160 * 1024;
}

hipError_t launch_lmhead_decode(int wdtype, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const int mt = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  if (wdtype == DEC_BF16) {
    if (mt == 1) return lmhead_go<DEC_BF16, 1>(a, s);
    if (mt == 2) return lmhead_go<DEC_BF16, 2>(a, s);
    return lmhead_go<DEC_BF16, 4>(a, s);
  }
  if (wdtype == DEC_UINT4_G32) {
    if (mt == 1) return lmhead_go<DEC_UINT4_G32, 1>(a, s);
    if (mt == 2) return lmhead_go<DEC_UINT4_G32, 2>(a, s);
    return lmhead_go<DEC_UINT4_G32, 4>(a, s);
  }
  if (wdtype == DEC_INT4_SYM_G32) {
    if (mt == 1) return lmhead_go<DEC_INT4_SYM_G32, 1>(a, s);
    if (mt == 2) return lmhead_go<DEC_INT4_SYM_G32, 2>(a, s);
    return lmhead_go<DEC_INT4_SYM_G32, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

// LDS bytes of the staged path: the activation rows (rpb) and, for bf16 weights, the weight
// rows (16 per matrix), or the wave partials if larger
template <int WF, int EPI, int MT>
static size_t decode_lds_bytes(int K, int rpb) {
  const size_t nb = EPI == EPI_SWIGLU ? 2 : 1;
  const size_t act = (size_t)rpb * K * 2 + (WF == DEC_BF16 && nb == 1 ? 16 * K * 2 : 0);
  const size_t part = (size_t)kDecWaves * nb * MT * 4 * 64 * 4;
  return act > part ? act : part;
}

template <int EPI>
static bool decode_staged(int K, size_t lds) {  // chunks per row a multiple of 16 (the swizzle), within LDS
  return (K * 2 / 16) % 16 == 0 && lds <= 159 * 1024;  // (1 KB left for the kernel's static LDS)
}

template <int WF, int EPI, int MT, int NKS, bool LDSA, int RPB>
static hipError_t gemm_decode_kernel_launch(const GemmArgs& a, int nw, dim3 g, size_t lds, hipStream_t s) {
  if constexpr (LDSA) {
    static size_t limit = 0;  // the dynamic LDS limit raised so far for this instantiation
    if (lds > limit) {
      hipError_t e = hipFuncSetAttribute((const void*)gemm_decode<WF, EPI, MT, NKS, true, RPB>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      limit = lds;
    }
  }
  launch_kernel(gemm_decode<WF, EPI, MT, NKS, LDSA, RPB>, g, dim3(512), (uint32_t)(LDSA ? lds : 0), s, a, nw);
  return hipGetLastError();
}

// rows8: blocks of 8 rows (RESID products with few column groups: four blocks per column tile,
// all on one XCD, so the tile's weights come from HBM once and from L2 after)
template <int WF, int EPI, int MT, int NKS>
static hipError_t gemm_decode_launch(const GemmArgs& a, int nw, bool rows8, hipStream_t s) {
  const size_t lds = decode_lds_bytes<WF, EPI, MT>(a.K, 16 * MT);
  if constexpr (EPI == EPI_RESID && MT == 1) {
    // (the MFMA tile reads activation rows 8..15 too: the allocation covers 16 rows)
    const size_t lds8 = std::max(decode_lds_bytes<WF, EPI, 1>(a.K, 8), (size_t)16 * a.K * 2);
    if (rows8 && decode_staged<EPI>(a.K, lds8))
      return gemm_decode_kernel_launch<WF, EPI, 1, NKS, true, 8>(a, nw, dim3((a.N + 15) / 16, (a.M + 7) / 8), lds8, s);
  }
  const dim3 g((a.N + 15) / 16, (a.M + 16 * MT - 1) / (16 * MT));
  if (decode_staged<EPI>(a.K, lds)) return gemm_decode_kernel_launch<WF, EPI, MT, NKS, true, 16 * MT>(a, nw, g, lds, s);
  return gemm_decode_kernel_launch<WF, EPI, MT, NKS, false, 16 * MT>(a, nw, g, lds, s);
}

template <int WF, int MT, int NKS>
static hipError_t gemm_decode_go(int epi, const GemmArgs& a, int nw, bool rows8, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return gemm_decode_launch<WF, EPI_STORE, MT, NKS>(a, nw, false, s);
    case EPI_RESID: return gemm_decode_launch<WF, EPI_RESID, MT, NKS>(a, nw, rows8, s);
    case EPI_SWIGLU: return gemm_decode_launch<WF, EPI_SWIGLU, MT, NKS>(a, nw, false, s);
  }
  return hipErrorInvalidValue;
}

template <int WF, int MT>
static hipError_t gemm_decode_nks(int epi, const GemmArgs& a, bool rows8, hipStream_t s) {
  // K split: nw waves of nks k-steps each, nw the largest of 8, 4, 2, 1 dividing K/32
  const int ksteps = a.K / 32;
  int nw = kDecWaves;
  while (ksteps % nw) nw >>= 1;
  switch (ksteps / nw) {
    case 1: return gemm_decode_go<WF, MT, 1>(epi, a, nw, rows8, s);
    case 2: return gemm_decode_go<WF, MT, 2>(epi, a, nw, rows8, s);
    case 3: return gemm_decode_go<WF, MT, 3>(epi, a, nw, rows8, s);
    case 4: return gemm_decode_go<WF, MT, 4>(epi, a, nw, rows8, s);
    case 6: return gemm_decode_go<WF, MT, 6>(epi, a, nw, rows8, s);
    case 8: return gemm_decode_go<WF, MT, 8>(epi, a, nw, rows8, s);
    case 12: return gemm_decode_go<WF, MT, 12>(epi, a, nw, rows8, s);
  }
  return hipErrorInvalidValue;
}

bool gemm_decode_supported(int wdtype, int K) {
  if (wdtype != DEC_BF16 && !is_q4(wdtype)) return false;
  const int ksteps = K / 32;
  int nw = kDecWaves;
  while (ksteps % nw) nw >>= 1;
  const int nks = ksteps / nw;
  return nks == 1 || nks == 2 || nks == 3 || nks == 4 || nks == 6 || nks == 8 || nks == 12;
}

hipError_t launch_gemm_decode(int wdtype, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  // blocks of 16 rows when M <= 16, when the product has few column groups (twice the blocks
  // then share the weights), or when only a 16-row activation tile fits in LDS; a row's result
  // is the same either way
  const size_t tile32 = (size_t)32 * a.K * 2;
  const bool rows16 = a.M <= 16 || (a.N + 15) / 16 < 128 || (tile32 > 128 * 1024 && tile32 / 2 <= 128 * 1024);
  const bool rows8 = epi == EPI_RESID && a.M > 8 && (a.N + 15) / 16 * ((a.M + 15) / 16) < 256;
  if (wdtype == DEC_BF16)
    return rows16 ? gemm_decode_nks<DEC_BF16, 1>(epi, a, rows8, s) : gemm_decode_nks<DEC_BF16, 2>(epi, a, rows8, s);
  if (wdtype == DEC_UINT4_G32)
    return rows16 ? gemm_decode_nks<DEC_UINT4_G32, 1>(epi, a, rows8, s)
                  : gemm_decode_nks<DEC_UINT4_G32, 2>(epi, a, rows8, s);
  if (wdtype == DEC_INT4_SYM_G32)
    return rows16 ? gemm_decode_nks<DEC_INT4_SYM_G32, 1>(epi, a, rows8, s)
                  : gemm_decode_nks<DEC_INT4_SYM_G32, 2>(epi, a, rows8, s);
  return hipErrorInvalidValue;
}

}  // namespace dec
