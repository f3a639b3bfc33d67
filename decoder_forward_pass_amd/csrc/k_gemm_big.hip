// Prefill projections as large MFMA tiles: C = A . W^T with W stored [out][in] ("Candle model
// runner" 2.4). A is the bf16 activation; W is bf16, or 4-bit dequantised while the tile is
// staged in LDS: uint4-g32 w = (q - zp) * scale ("Byte-identical...", "The bar we set") or
// symmetric int4-g32 w = q * scale ("Candle model runner" 2.5), rounded to bf16.
//
// Tiling: a block of 8 waves computes a 256 x 256 tile of C (waves 4 x 2, 64 x 128 each), or,
// for bf16 products whose 256 x 256 grid would not fill the chip, a 128 x 128 tile (waves 4 x 2,
// 32 x 64 each; the same loop with half the loads per wave and a 64 KB ring). bf16
// weights: both operands go from memory straight into LDS (direct-to-LDS loads) in K steps of
// 32 through a ring of four stages, three steps in flight, one barrier per step. 4-bit weights:
// K steps of 64, the next step's operands loaded into registers (and dequantised) while the
// current step's LDS copy feeds the MFMAs (two LDS stages, one barrier per step). Every output
// element is accumulated by v_mfma_f32_32x32x16_bf16 (the full-rate bf16 shape on this chip;
// the 16x16x32 shape issues at half the rate) over K in ascending order into a single
// accumulator, exactly as in the 64 x 64 tile kernel, so both give identical results and a
// row's result does not depend on M or on the other rows.
//
// Block order: the hardware deals consecutive block ids to the chip's 8 L2 domains in turn;
// the id is remapped so that each domain receives a contiguous run of tiles, walked 8 M tiles
// at a time, so concurrently running blocks share their A rows and W rows in one L2.
//
// Epilogues: store, residual add, SwiGLU (silu on the gate only, "Candle model runner" 2.4),
// and the attention input ("A real model in our own decoder", switch 5, and "Which channels
// rotate together"): per-head RMSNorm over head_dim with the layer's q_norm / k_norm gains,
// then the rotation of channel pairs (j, j + D/2) by pos * base^(-2j/D), q stored in the KV
// format, K and V written to the pool at block table[pos / B], slot pos % B ("Candle model
// runner" section 3, "Where a key lands"). A wave's 128 columns hold whole heads and channels
// j and j + D/2 of a head sit in the same lane, so this is all done in registers.
#include "kernels.h"

#include <utility>

namespace dec {

namespace {

constexpr int kBT = 256;            // block tile rows and columns
constexpr int kBK = 64;             // K per step (4-bit weights: register staging)
constexpr int kLR = kBK + 8;        // LDS row stride in bf16 (padded: conflict-free fragment reads)
constexpr int kStage = kBT * kLR;   // bf16 elements of one operand tile
constexpr size_t kBigLds = (size_t)2 * 2 * kStage * 2;  // two stages of A and B, bytes
// bf16 weights: direct-to-LDS staging, K steps of 32 in a ring of 4 stages (3 in flight);
// a stage holds 256 rows of 32 bf16 (64 B) of A, then of B; row r keeps its 16-byte chunk c at
// position c ^ ((r / 4) % 4), so the 16 rows of a fragment read fall on distinct banks
constexpr int kDK = 32, kDStages = 4;

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), expanded at compile time so
// that accumulator indices are constants (an unroll the optimizer may decline)
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

struct BigRowsB {
  const uint16_t* p[4];  // bf16: the thread's four B rows
};

}  // namespace

// The epilogue of a block's tile from its waves' accumulators: wave (wm, wn) holds rows
// m0 + 32 NBI wm .. + 32 NBI (NBI blocks of 32) and the NBJ 32-column blocks of brow_of.
template <int WF, int EPI, int D, bool KV_F16, int NBI, int NBJ>
__device__ __forceinline__ void big_epilogue(const GemmArgs& a, const QkRopeArgs& qk, f32x16 (&acc)[NBI][NBJ], int m0,
                                             int n0, int wm, int wn, int lane, const int* s_pos,
                                             const int64_t* s_blk) {
  static_assert(EPI != EPI_QKV || NBJ == 4, "Q|K|V epilogue: 128 columns (whole heads) per wave");
  // lane holds column fr of each 32 x 32 block, rows 8 g + 4 (lane / 32) + r
  const int fr = lane & 31;
  const int M = a.M;
  const int rbase = m0 + wm * (32 * NBI) + (lane >> 5) * 4;
  auto row_of = [&](int bi, int i) { return rbase + bi * 32 + 8 * (i >> 2) + (i & 3); };
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    // per 32 x 32 block: the 16 residual values are all requested before any is updated
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
      for (int bj = 0; bj < NBJ; ++bj) {
        const int n = n0 + wn * (32 * NBJ) + bj * 32 + fr;
        const int nc = min(n, a.N - 1);
        float xo[16];
        if constexpr (EPI == EPI_RESID) {
#pragma unroll
          for (int i = 0; i < 16; ++i) xo[i] = ((const float*)a.C)[(int64_t)min(row_of(bi, i), M - 1) * a.ldc + nc];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = row_of(bi, i);
          if (m < M && n < a.N) {
            float* c = (float*)a.C + (int64_t)m * a.ldc + n;
            if constexpr (EPI == EPI_STORE)
              *c = acc[bi][bj][i];
            else
              *c = xo[i] + acc[bi][bj][i];
          }
        }
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = row_of(bi, i);
        if (m >= M) continue;
#pragma unroll
        for (int bj = 0; bj < NBJ / 2; ++bj) {
          const int f = n0 + wn * (16 * NBJ) + bj * 32 + fr;
          if (f >= a.N) continue;
          const float g = acc[bi][bj][i], u = acc[bi][bj + NBJ / 2][i];
          const float y = silu_mul(g, u);
          if (a.c_bf16)
            ((uint16_t*)a.C)[(int64_t)m * a.ldc + f] = f32_to_bf16_bits(y);
          else
            ((float*)a.C)[(int64_t)m * a.ldc + f] = y;
        }
      }
  } else {
    // Q|K|V: heads of D channels; a head spans BPH 32-column blocks, HPW heads per wave
    constexpr int BPH = D >= 32 ? D / 32 : 1, HPW = 128 / D, HALF = D / 2;
    const int H = qk.n_heads, Hkv = qk.n_kv_heads;
    const int hw0 = (n0 + wn * 128) / D;  // global head index of the wave's first head
    // this lane's channels of a head are b * 32 + fr (D = 32: fr); their q and k gains
    float gq[BPH], gk[BPH];
#pragma unroll
    for (int b = 0; b < BPH; ++b) {
      gq[b] = qk.q_norm[b * 32 + fr];
      gk[b] = qk.k_norm[b * 32 + fr];
    }
    // Rows in batches of 8 (2 NBI batches): the next batch's positions, blocks and rotation
    // factors are requested before the current batch is normalised, rotated and stored, so the
    // rotation table's latency is paid once rather than once per batch
    constexpr int NCS = D >= 64 ? BPH / 2 : 1;
    struct Rows {
      float2 cs[8][NCS];  // (the rows' positions and blocks are read again from LDS)
    };
    auto fetch = [&](auto q_c, Rows& rw) __attribute__((always_inline)) {
      constexpr int bi = decltype(q_c)::value >> 1, i0 = (decltype(q_c)::value & 1) * 8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int pos = s_pos[row_of(bi, i0 + r) - m0];
#pragma unroll
        for (int b = 0; b < NCS; ++b)
          rw.cs[r][b] = qk.rope[(int64_t)pos * HALF + (D >= 64 ? b * 32 + fr : (fr & 15))];
      }
    };
    auto work = [&](auto q_c, const Rows& rw) __attribute__((always_inline)) {
      constexpr int bi = decltype(q_c)::value >> 1, i0 = (decltype(q_c)::value & 1) * 8;
      int pos_r[8];
      int64_t blk_r[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int lr = row_of(bi, i0 + r) - m0;
        pos_r[r] = s_pos[lr];
        blk_r[r] = s_blk[lr];
      }
      const float2 (&cs_r)[8][NCS] = rw.cs;
      static_for<8>([&](auto r_c) {
        constexpr int r = decltype(r_c)::value, i = i0 + r;
        const int m = row_of(bi, i);
        const int64_t blk = blk_r[r];
        const int slot = pos_r[r] & (qk.pool.block_tokens - 1);
        static_for<HPW>([&](auto hw_c) {
          constexpr int hw = decltype(hw_c)::value;
          const int hh = hw0 + hw;  // wave-uniform
          if (hh >= H + 2 * Hkv) return;
          float v[BPH];
#pragma unroll
          for (int b = 0; b < BPH; ++b) v[b] = acc[bi][(hw * D) / 32 + b][i];
          if (hh < H + Hkv) {
            // RMSNorm over the head's D channels: BPH blocks in the lane, then 32 lanes
            float ss = 0.f;
#pragma unroll
            for (int b = 0; b < BPH; ++b) ss += v[b] * v[b];
            ss = group_sum<32>(ss);
            const float inv = __builtin_amdgcn_rsqf(ss / (float)D + qk.eps);  // (hardware rsqrt, within an ulp)
            const bool isq = hh < H;
            if constexpr (D >= 64) {
#pragma unroll
              for (int b = 0; b < BPH / 2; ++b) {
                const float2 cs = cs_r[r][b];
                const float x1 = v[b] * inv * (isq ? gq[b] : gk[b]);
                const float x2 = v[b + BPH / 2] * inv * (isq ? gq[b + BPH / 2] : gk[b + BPH / 2]);
                v[b] = x1 * cs.x - x2 * cs.y;
                v[b + BPH / 2] = x2 * cs.x + x1 * cs.y;
              }
            } else {
              // D = 32: the head is one block; channel fr pairs with channel fr ^ 16, held by
              // the lane 16 away
              const float2 cs = cs_r[r][0];
              const float xs = v[0] * inv * (isq ? gq[0] : gk[0]);
              const float xo = __shfl_xor(xs, 16, 64);
              v[0] = fr < 16 ? xs * cs.x - xo * cs.y : xs * cs.x + xo * cs.y;
            }
          }
          if (m >= M) return;
          if (hh < H) {
            const int64_t o = ((int64_t)m * H + hh) * D + fr;
#pragma unroll
            for (int b = 0; b < BPH; ++b) {
              if constexpr (KV_F16)
                ((uint16_t*)qk.q_out)[o + b * 32] = f32_to_f16_bits(v[b]);
              else
                ((float*)qk.q_out)[o + b * 32] = v[b];
            }
          } else {
            const int kv = hh < H + Hkv ? 0 : 1;
            const int kvh = hh - H - kv * Hkv;
            const int64_t o = qk.pool.offset(qk.layer, kv, blk, kvh, slot) + fr;
#pragma unroll
            for (int b = 0; b < BPH; ++b) {
              if constexpr (KV_F16)
                ((uint16_t*)qk.pool.base)[o + b * 32] = f32_to_f16_bits(v[b]);
              else
                ((float*)qk.pool.base)[o + b * 32] = v[b];
            }
          }
        });
      });
    };
    Rows ra, rb;
    fetch(std::integral_constant<int, 0>{}, ra);
    static_for<2 * NBI>([&](auto q_c) {
      constexpr int q = decltype(q_c)::value;
      if constexpr (q + 1 < 2 * NBI) fetch(std::integral_constant<int, q + 1>{}, (q & 1) ? ra : rb);
      work(q_c, (q & 1) ? rb : ra);
    });
  }
}

template <int WF, int EPI, int D, bool KV_F16, int TS>
__global__ __launch_bounds__(512) void gemm_big(GemmArgs a, QkRopeArgs qk) {
  // TS x TS tiles: 256 (every format and epilogue), or 128 (bf16 weights; store, residual and
  // SwiGLU epilogues) for grids of 256-tiles too small to fill the chip. Waves 4 x 2, each
  // TS / 4 rows (NBI blocks of 32) by TS / 2 columns (NBJ blocks of 32).
  static_assert(TS == 256 || (TS == 128 && WF == DEC_BF16 && EPI != EPI_QKV), "128-tiles: bf16, no Q|K|V");
  constexpr int NBI = TS / 128, NBJ = TS / 64;
  constexpr int TN = EPI == EPI_SWIGLU ? TS / 2 : TS;  // output columns (features) per tile
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [stage][A | B][TS][row]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int M = a.M, K = a.K;
  const int mt_n = (M + TS - 1) / TS;
  const int nt_n = (a.N + TN - 1) / TN;

  // ---- block id -> tile (contiguous runs per L2 domain, 8 M tiles per group)
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  if (nblk % 8 == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
  const int gsz = 8 * nt_n;
  const int grp = bid / gsz, gm0 = grp * 8, gmn = min(8, mt_n - gm0);
  const int tm = gm0 + (bid % gsz) % gmn, tn = (bid % gsz) / gmn;
  const int m0 = tm * TS;
  const int n0 = tn * TN;

  // Q|K|V: position and pool block of each of the tile's rows, fetched once up front (the
  // barriers of the main loop publish them)
  __shared__ int s_pos[EPI == EPI_QKV ? TS : 1];
  __shared__ int64_t s_blk[EPI == EPI_QKV ? TS : 1];
  if constexpr (EPI == EPI_QKV) {
    if (tid < TS) {
      const int mc = min(m0 + tid, M - 1);
      const int pos = qk.b.row_pos[mc];
      s_pos[tid] = pos;
      s_blk[tid] = qk.b.block_tables[(int64_t)qk.b.row_seq[mc] * qk.b.tbl_stride + (pos >> qk.pool.block_shift)];
    }
  }

  // ---- per-thread staging sources: A and B chunks of 16 B (8 bf16), rows tid/8 + 64 i
  const int srow = tid >> 3, sc8 = tid & 7;
  const uint16_t* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ap[i] = (const uint16_t*)a.A + (int64_t)min(m0 + srow + 64 * i, M - 1) * a.lda + sc8 * 8;
  // B row of LDS row r: SwiGLU rows 0..TS/2-1 gate, TS/2..TS-1 up (features n0 + r % (TS/2));
  // otherwise row n0 + r of the Q|K|V (or single) concatenation
  // (segments are selected with constant indices, so the arguments stay in registers)
  auto b_src = [&](int r, int& rr) -> WMat {
    if constexpr (EPI == EPI_SWIGLU) {
      const WMat m = r < TS / 2 ? a.seg[0] : a.seg[1];
      rr = min(n0 + (r & (TS / 2 - 1)), m.rows - 1);
      return m;
    } else {
      int n = min(n0 + r, a.N - 1);
      if (a.nseg > 1 && n >= a.seg[0].rows) {
        n -= a.seg[0].rows;
        if (a.nseg > 2 && n >= a.seg[1].rows) {
          rr = n - a.seg[1].rows;
          return a.seg[2];
        }
        rr = n;
        return a.seg[1];
      }
      rr = n;
      return a.seg[0];
    }
  };
  BigRowsB bp;
  const uint8_t* qcodes = nullptr;
  const uint16_t *qscale = nullptr, *qzp = nullptr;  // (the signed format has no zero point)
  const int urow = tid >> 1, uhalf = tid & 1;  // 4-bit: a thread dequantises 32 k of one row
  if constexpr (WF == DEC_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int rr;
      const WMat m = b_src(srow + 64 * i, rr);
      bp.p[i] = (const uint16_t*)m.w + (int64_t)rr * K + sc8 * 8;
    }
  } else {
    int rr;
    const WMat m = b_src(urow, rr);
    qcodes = (const uint8_t*)m.w + (int64_t)rr * (K / 2) + uhalf * 16;
    qscale = m.scale + (int64_t)rr * (K / 32) + uhalf;
    if constexpr (WF == DEC_UINT4_G32) qzp = m.zp + (int64_t)rr * (K / 32) + uhalf;
  }

  u32x4 ra[4], rb[4];
  uint32_t rsz = 0;  // 4-bit: scale | zp << 16 (uint4)
  auto load_step = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = *(const u32x4*)(ap[i] + k0);
    if constexpr (WF == DEC_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = *(const u32x4*)(bp.p[i] + k0);
    } else {
      rb[0] = *(const u32x4*)(qcodes + k0 / 2);
      rsz = (uint32_t)qscale[k0 / 32];
      if constexpr (WF == DEC_UINT4_G32) rsz |= (uint32_t)qzp[k0 / 32] << 16;
    }
  };
  auto store_step = [&](int st) {
    uint16_t* As = lds + (size_t)st * 2 * kStage;
    uint16_t* Bs = As + kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(As + (srow + 64 * i) * kLR + sc8 * 8) = ra[i];
    if constexpr (WF == DEC_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4*)(Bs + (srow + 64 * i) * kLR + sc8 * 8) = rb[i];
    } else {
      const float sc = q4_scale<WF>(rsz & 0xffffu);
      float zp;
      if constexpr (WF == DEC_UINT4_G32)
        zp = bf16_bits_to_f32(rsz >> 16);
      else
        zp = 8.0f;  // signed nibbles read with their top bit flipped
      uint16_t* d = Bs + urow * kLR + uhalf * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t byte = (q4_codes<WF>(rb[0][q]) >> (8 * j)) & 0xffu;
          w[j] = pack_bf16x2(dequant_u4(byte & 15u, zp, sc), dequant_u4(byte >> 4, zp, sc));
        }
        *(u32x4*)(d + q * 8) = w;
      }
    }
  };

  // LDS row of the wave's 32-column block bj (SwiGLU: the first NBJ / 2 blocks gate, the others
  // up, same features)
  auto brow_of = [&](int bj) {
    if constexpr (EPI == EPI_SWIGLU)
      return (bj / (NBJ / 2)) * (TS / 2) + wn * (16 * NBJ) + (bj % (NBJ / 2)) * 32;
    else
      return wn * (32 * NBJ) + bj * 32;
  };

  // v_mfma_f32_32x32x16_bf16: operand lane l holds row l % 32, k = 8 * (l / 32) .. +8;
  // accumulator register i of lane l is row 8 * (i / 4) + 4 * (l / 32) + i % 4, column l % 32
  f32x16 acc[NBI][NBJ];
#pragma unroll
  for (int i = 0; i < NBI; ++i)
#pragma unroll
    for (int j = 0; j < NBJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto mfma_step = [&](const bf16x8 (&af)[NBI], const bf16x8 (&bf)[NBJ]) {
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
      for (int bj = 0; bj < NBJ; ++bj)
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[bi], bf[bj], acc[bi][bj], 0, 0, 0);
  };
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  if constexpr (WF == DEC_BF16) {
    // Waves 0-3 stage the A rows, waves 4-7 the B rows, TS / 4 rows per wave in LPW 1 KB
    // direct-to-LDS loads per K step (16 rows of 64 B; lane l fills row l / 4, position l % 4,
    // from the source chunk that position holds). The loads of three K steps are in flight.
    constexpr int LPW = TS / 64, STG = 2 * TS * kDK;  // loads per wave per step; bf16 per stage
    const int nkd = K / kDK;
    const int opb = wave >> 2, wq = wave & 3;
    const int lc = (lane & 3) ^ ((lane >> 4) & 3);
    const uint16_t* dsrc[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = wq * (TS / 4) + i * 16 + (lane >> 2);
      if (opb == 0) {
        dsrc[i] = (const uint16_t*)a.A + (int64_t)min(m0 + r, M - 1) * a.lda + lc * 8;
      } else {
        int rr;
        const WMat m = b_src(r, rr);
        dsrc[i] = (const uint16_t*)m.w + (int64_t)rr * K + lc * 8;
      }
    }
    uint16_t* const dbase = lds + opb * TS * kDK + wq * (TS / 4) * kDK;
    auto dma = [&](int t) {
      uint16_t* d = dbase + (t & (kDStages - 1)) * STG;
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(dsrc[i] + t * kDK),
                                         (void __attribute__((address_space(3)))*)(d + i * 16 * kDK), 16, 0, 0);
    };
    // fragment (row, k-step ks) of a staged operand: chunk 2 ks + lane / 32 of the row
    const int fsw = (fr >> 2) & 3;
    auto dfrag = [&](const uint16_t* S, int row, int ks) {
      return __builtin_bit_cast(bf16x8, *(const u32x4*)(S + row * kDK + (((ks * 2 + (lane >> 5)) ^ fsw) * 8)));
    };
    // Fragments of step t + 1 are read from LDS while step t's MFMAs run (two register sets,
    // used in turn; K / 32 is even); the loads of the three steps after t + 1 are in flight.
    struct Frags {
      bf16x8 a[2][NBI], b[2][NBJ];
    };
    auto read = [&](int t, Frags& f) __attribute__((always_inline)) {
      const uint16_t* As = lds + (t & (kDStages - 1)) * STG;
      const uint16_t* Bs = As + TS * kDK;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int bi = 0; bi < NBI; ++bi) f.a[ks][bi] = dfrag(As, wm * (32 * NBI) + bi * 32 + fr, ks);
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) f.b[ks][bj] = dfrag(Bs, brow_of(bj) + fr, ks);
      }
    };
    dma(0);
    if (nkd > 1) dma(1);
    if (nkd > 2) dma(2);
    if (nkd > 3) dma(3);
    // stage 0 has landed for this wave once at most the later stages' loads are outstanding
    if (nkd > 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LPW) : "memory");
    else if (nkd > 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW) : "memory");
    else if (nkd > 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    Frags fa, fb;
    read(0, fa);
    auto step = [&](int t, const Frags& cur, Frags& nxt) __attribute__((always_inline)) {
      // stage t + 1 has landed for this wave (the stages after it, up to t + 3, may be in
      // flight) and this wave's reads of stage t are done; the barrier then publishes stage
      // t + 1 and frees stage t for the loads of step t + 4. A plain s_barrier: the workgroup
      // fence of __syncthreads would also wait for the loads still in flight.
      const int later = min(nkd - 1, t + 3) - (t + 1);
      if (later >= 2)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * LPW) : "memory");
      else if (later == 1)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LPW) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + 4 < nkd) dma(t + 4);
      read(min(t + 1, nkd - 1), nxt);  // (the last step reads its own stage again, unused)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) mfma_step(cur.a[ks], cur.b[ks]);
      // the fragment reads spread between the matrix instructions (NR reads, NM MFMAs: one or
      // two reads before each MFMA), so the reads complete under them
      constexpr int NR = 2 * (NBI + NBJ), NM = 2 * NBI * NBJ;
      static_for<NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int nr = NR >= NM ? NR / NM + (i < NR % NM ? 1 : 0) : (i < NR ? 1 : 0);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      });
    };
    for (int t = 0; t < nkd; t += 2) {
      step(t, fa, fb);
      step(t + 1, fb, fa);
    }
  } else {
  const int nk = K / kBK;
  constexpr int NKS = kBK / 16;  // MFMA k-steps per K step
  // fragments of k-step ks of the LDS stage st
  auto read_frags = [&](int st, int ks, bf16x8 (&af)[2], bf16x8 (&bf)[4]) {
    const uint16_t* As = lds + (size_t)st * 2 * kStage;
    const uint16_t* Bs = As + kStage;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
      af[bi] = __builtin_bit_cast(bf16x8, *(const u32x4*)(As + (wm * 64 + bi * 32 + fr) * kLR + ks * 16 + fk));
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
      bf[bj] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Bs + (brow_of(bj) + fr) * kLR + ks * 16 + fk));
  };

  // Pipeline: the fragments of the next k-step are read from LDS while the current k-step's
  // MFMAs run (two fragment sets). The next K step's operands are loaded from memory during
  // the first k-steps, written to the other LDS stage before the last k-step, and published
  // by the barrier, so the last k-step's MFMAs cover the first reads of the next stage.
  bf16x8 fa[2][2], fb[2][4];
  load_step(0);
  store_step(0);
  __syncthreads();
  read_frags(0, 0, fa[0], fb[0]);
  for (int t = 0; t < nk; ++t) {
    const int st = t & 1;
    const bool more = t + 1 < nk;
    if (more) load_step((t + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < NKS - 1; ++ks) {
      read_frags(st, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      mfma_step(fa[ks & 1], fb[ks & 1]);
    }
    if (more) store_step(st ^ 1);
    __syncthreads();
    if (more) read_frags(st ^ 1, 0, fa[NKS & 1], fb[NKS & 1]);
    mfma_step(fa[(NKS - 1) & 1], fb[(NKS - 1) & 1]);
  }
  }

  big_epilogue<WF, EPI, D, KV_F16, NBI, NBJ>(a, qk, acc, m0, n0, wm, wn, lane, s_pos, s_blk);
}

template <int WF, int EPI, int D, bool KV_F16, int TS = 256>
static hipError_t big_go(const GemmArgs& a, const QkRopeArgs& qk, hipStream_t s) {
  const size_t lds = WF == DEC_BF16 ? (size_t)kDStages * 2 * TS * kDK * 2 : kBigLds;
  static bool attr = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_big<WF, EPI, D, KV_F16, TS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int tn = EPI == EPI_SWIGLU ? TS / 2 : TS;
  const int mt = (a.M + TS - 1) / TS;
  const int nt = (a.N + tn - 1) / tn;
  launch_kernel(gemm_big<WF, EPI, D, KV_F16, TS>, dim3(mt * nt), dim3(512), (uint32_t)lds, s, a, qk);
  return hipGetLastError();
}

template <int WF>
static hipError_t big_epi(int epi, const GemmArgs& a, const QkRopeArgs* qk, hipStream_t s) {
  const QkRopeArgs none{};
  switch (epi) {
    case EPI_STORE: return big_go<WF, EPI_STORE, 128, false>(a, none, s);
    case EPI_RESID: return big_go<WF, EPI_RESID, 128, false>(a, none, s);
    case EPI_SWIGLU: return big_go<WF, EPI_SWIGLU, 128, false>(a, none, s);
    case EPI_QKV:
      if (!qk) return hipErrorInvalidValue;
      switch (qk->head_dim) {
        case 32: return qk->kv_f16 ? big_go<WF, EPI_QKV, 32, true>(a, *qk, s) : big_go<WF, EPI_QKV, 32, false>(a, *qk, s);
        case 64: return qk->kv_f16 ? big_go<WF, EPI_QKV, 64, true>(a, *qk, s) : big_go<WF, EPI_QKV, 64, false>(a, *qk, s);
        case 128:
          return qk->kv_f16 ? big_go<WF, EPI_QKV, 128, true>(a, *qk, s) : big_go<WF, EPI_QKV, 128, false>(a, *qk, s);
      }
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

bool gemm_big_supported(int wdtype, int epi, int head_dim) {
  if (wdtype != DEC_BF16 && !is_q4(wdtype)) return false;
  if (epi == EPI_QKV) return head_dim == 32 || head_dim == 64 || head_dim == 128;
  return epi == EPI_STORE || epi == EPI_RESID || epi == EPI_SWIGLU;
}

hipError_t launch_gemm_big(int wdtype, int epi, const GemmArgs& a, const QkRopeArgs* qk, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % kBK) return hipErrorInvalidValue;
  if (wdtype == DEC_BF16) return big_epi<DEC_BF16>(epi, a, qk, s);
  if (wdtype == DEC_UINT4_G32) return big_epi<DEC_UINT4_G32>(epi, a, qk, s);
  if (wdtype == DEC_INT4_SYM_G32) return big_epi<DEC_INT4_SYM_G32>(epi, a, qk, s);
  return hipErrorInvalidValue;
}

bool gemm_mid_supported(int wdtype, int epi) {
  return wdtype == DEC_BF16 && (epi == EPI_STORE || epi == EPI_RESID || epi == EPI_SWIGLU);
}

hipError_t launch_gemm_mid(int wdtype, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!gemm_mid_supported(wdtype, epi) || a.K % kBK) return hipErrorInvalidValue;
  const QkRopeArgs none{};
  switch (epi) {
    case EPI_STORE: return big_go<DEC_BF16, EPI_STORE, 128, false, 128>(a, none, s);
    case EPI_RESID: return big_go<DEC_BF16, EPI_RESID, 128, false, 128>(a, none, s);
    default: return big_go<DEC_BF16, EPI_SWIGLU, 128, false, 128>(a, none, s);
  }
}

}  // namespace dec
