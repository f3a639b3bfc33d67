// Causal grouped-query attention of prefill rows over the paged KV pool, on MFMA
// ("Candle model runner" 2.4, second equation): the flash-style kernel for an f16 pool.
// The other attention paths (rows + combine, decode) are in k_attn.hip.
#include "kernels.h"

namespace dec {

// ---- flash-style prefill attention (f16 pool, MFMA) ----------------------------------------
// Causal attention of one sequence's new rows over its paged keys ("Candle model runner" 2.4,
// second equation; keys up to and including the query's absolute position), read in place from
// the pool. A block has 4 waves of 32 query positions: one head and 128 positions (one-head
// groups), or two heads and 64 positions (two-head groups, a 128-position query tile split over
// two blocks). Two blocks share a compute unit and run out of step, so one's matrix products
// overlap the other's softmax. Key tiles of 64 positions, aligned to position 0 of the
// sequence, are staged in LDS by direct-to-LDS loads, two tiles of K and two of V; while tile
// t is finished, S^T of tile t + 1 is computed and the next tiles load. Per key tile and
// wave, with v_mfma_f32_32x32x16_f16:
//   S^T = K . Q^T (keys x queries), scaled into the exp2 domain and causally masked;
//   online softmax per query (a query's 64 scores sit in lanes l and l ^ 32);
//   O^T += V^T . P^T, where P^T is taken from the S^T accumulators as they are: a lane's eight
//   k-slots of k-step s stand for keys 16 s + 8 (j / 4) + 4 (l / 32) + j % 4, a fixed
//   relabelling of the summation index applied to both operands. V stays row-major in LDS;
//   gfx950's transposing LDS read (ds_read_b64_tr_b16) hands each lane four consecutive keys
//   of its channel.
// A query sees the key tiles 0 .. floor(pos / 64) in order; a later, fully masked tile leaves
// its state unchanged bit for bit (scale exp2(0) = 1, weights exp2(-inf) = 0, masked values
// zero). The result therefore does not depend on how queries are grouped into tiles, so
// batched, chunked and single-shot prefill agree exactly.

namespace {
constexpr int kPfKT = 64;  // keys per tile
// LDS tiles: K or V of 64 keys, [64 keys][D] row-major f16. The 16-byte chunk c of row r is
// stored at chunk position c ^ f(r), so that the fragment reads meet no bank conflict: fk for
// K (the 16 rows of a 16-byte-per-lane read pass at one chunk index), fv for V (the 4 rows x 4
// chunks of a transposing read pass).
template <int D>
struct PrefillLds {
  static constexpr int ROWB = 2 * D;              // bytes per key row
  static constexpr int TILEB = kPfKT * ROWB;      // one tile
  static constexpr int NC = D / 8;                // 16-byte chunks per row
  static constexpr int RPW = 16 / NC;             // rows per 256-byte bank window
  static constexpr int RPI = 1024 / ROWB;         // rows per 1 KB direct-to-LDS load of a wave
  static constexpr int NI = 16 / RPI;             // such loads per wave and matrix (16 rows each)
  __device__ static int fk(int r) { return (r / RPW) % NC; }
  __device__ static int fv(int r) { return RPW < 4 ? 4 * ((r / RPW) % (4 / RPW)) : 0; }
};
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// the reference maximum of a query moves only past this margin (log2 units: weights <= 256)
constexpr float kLag = 8.0f;
// max / sum of a value and its partner 32 lanes away (gfx950 row swap: no LDS round trip;
// both operations are commutative, so both lanes get the same bits)
__device__ __forceinline__ float swap_halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
}  // namespace

template <int D, int G, int SPLIT, bool BF16_OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_prefill_kernel(AttnPrefillArgs a) {
  using L = PrefillLds<D>;
  constexpr int KT = kPfKT, QT = kPrefillQueryTile;
  constexpr int WPH = 4 / SPLIT;           // waves per head
  constexpr int QB = QT / SPLIT;           // query positions per block
  constexpr int ROWB = L::ROWB;
  constexpr int NDS = D / 16;              // k-steps of S^T over the head dimension
  constexpr int NDB = D / 32;              // 32-row blocks of O^T
  static_assert(QT == 128 && SPLIT == G && WPH * G == 4, "4 waves of 32 query positions per block");
  static_assert(D == 32 || D == 64 || D == 128, "head dimension");
  // two K tiles and two V tiles, as four arrays: the compiler then knows that a tile being read
  // is not the one being loaded, and places no wait for the loads before the reads
  __shared__ __attribute__((aligned(16))) char ks0[L::TILEB], ks1[L::TILEB], vs0[L::TILEB], vs1[L::TILEB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  const int gh = wave / WPH, qsub = wave % WPH;
  const int kvh = blockIdx.x, tile = blockIdx.y / SPLIT, qb0 = (blockIdx.y % SPLIT) * QB;
  const int seq = a.b.tiles[2 * tile], row0 = a.b.tiles[2 * tile + 1];
  const int s_start = a.b.seq_start[seq], s_n = a.b.seq_nnew[seq], s_row0 = a.b.seq_row0[seq];
  const int ctx_end = s_start + s_n;
  const int p0 = s_start + (row0 - s_row0);
  const int tile_rows = min(QT, s_n - (row0 - s_row0));
  if (qb0 >= tile_rows) return;  // (a ragged last tile: this block has no query; block-uniform)
  const int pmax = p0 + min(qb0 + QB, tile_rows) - 1;  // the block's last query position
  const int H = a.n_heads;
  const int bsh = a.pool.block_shift, bmask = a.pool.block_tokens - 1;
  // the table is not written while the kernel runs: read it through the scalar cache
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(a.b.block_tables + (int64_t)seq * a.b.tbl_stride);
  const int64_t slab_b = (int64_t)a.n_kv_heads * a.pool.block_tokens * ROWB;  // bytes per pool block
  const char* kbase = (const char*)a.pool.base + (int64_t)a.layer * 2 * a.pool.n_blocks * slab_b +
                      (int64_t)kvh * a.pool.block_tokens * ROWB;
  const char* vbase = kbase + a.pool.n_blocks * slab_b;
  const int head = kvh * G + gh;

  // this lane's query (column of S^T and O^T)
  const int qi = qb0 + qsub * 32 + ql;
  const bool qvalid = qi < tile_rows;
  const int qrow = row0 + min(qi, tile_rows - 1);
  const int qpos = p0 + qi;
  const int wq0 = p0 + qb0 + qsub * 32;  // the wave's first query position
  f16x8 qf[NDS];
#pragma unroll
  for (int ks = 0; ks < NDS; ++ks)
    qf[ks] = __builtin_bit_cast(f16x8, *(const u32x4*)(a.q + ((int64_t)qrow * H + head) * D + ks * 16 + hl * 8));

  // ---- staging. Wave w loads rows 16 w .. 16 w + 15 of the K and V tiles (in one pool block,
  // since blocks hold at least 16 positions) with 1 KB direct-to-LDS loads through a buffer
  // descriptor whose range ends at the context's last key: rows past it (and a whole tile past
  // the block's last query) arrive as zeros, and nothing outside the block is read. Lane l of
  // load i fills row i * RPI + l / NC at chunk position l % NC, so it reads the chunk that
  // position stands for.
  const int last_key = ctx_end - 1;
  uint32_t dk[L::NI], dv[L::NI];
#pragma unroll
  for (int i = 0; i < L::NI; ++i) {
    const int x = i * L::RPI + lane / L::NC, pc = lane % L::NC;
    dk[i] = x * ROWB + ((pc ^ L::fk(x)) * 16);
    dv[i] = x * ROWB + ((pc ^ L::fv(x)) * 16);
  }
  auto block_id = [&](int kt) { return table[min(kt * KT + 16 * wave, last_key) >> bsh]; };
  // rows 16 w .. 16 w + 15 of key tile kt of one matrix into an LDS tile
  auto dma = [&](const char* base, int kt, int blk, char* dst, bool live, const uint32_t (&dof)[L::NI]) {
    const int r0 = kt * KT + 16 * wave;
    // (wave-uniform; made explicit so that the descriptor stays in scalar registers)
    const int rows = __builtin_amdgcn_readfirstlane(live ? min(max(last_key + 1 - r0, 0), 16) : 0);
    const int64_t off = (int64_t)blk * slab_b + (int64_t)(r0 & bmask) * ROWB;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), 0, rows * ROWB, 0x00020000);
    char* d = dst + 16 * wave * ROWB;
#pragma unroll
    for (int i = 0; i < L::NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void __attribute__((address_space(3)))*)(d + i * 1024), 16, (int)dof[i], 0, 0, 0);
  };

  // fragment read offsets within a tile. K: lane (ql, hl) reads row 32 kb + ql, chunk
  // 2 ks + hl. V (transposing read): lane l supplies row 16 s + 8 h + 4 (l / 32) + (l / 4) % 4
  // at channels 32 db + 16 ((l / 16) % 2) + 4 (l % 4) .. + 3 and receives channel 32 db + ql of
  // that group of four rows.
  uint32_t ka[NDS], va[NDB];
#pragma unroll
  for (int ks = 0; ks < NDS; ++ks) ka[ks] = ql * ROWB + (((2 * ks + hl) ^ L::fk(ql)) * 16);
  {
    const int g = lane >> 4, jj = (lane >> 2) & 3, t = lane & 3;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      va[db] = (4 * (g >> 1) + jj) * ROWB + (((db * 4 + 2 * (g & 1) + (t >> 1)) ^ L::fv(jj)) * 16) + (t & 1) * 8;
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m = -__builtin_inff(), l = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const int n_kt = pmax / KT + 1;

  // S^T = K . Q^T for a tile's 64 keys (two 32-key blocks)
  auto scores = [&](const char* Ks, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NDS; ++ks) {
        const f16x8 kf = __builtin_bit_cast(f16x8, *(const u32x4*)(Ks + kb * 32 * ROWB + ka[ks]));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sacc[kb], 0, 0, 0);
      }
    }
  };
  // online softmax of this lane's query over tile kt, then O^T += V^T . P^T. Only a tile that
  // reaches past the wave's first query position needs the causal mask; elsewhere every key
  // is visible. The tile maximum is taken over the raw scores and scaled afterwards (scaling
  // by a positive constant is monotone under rounding, so this is the maximum of the scaled
  // scores). The reference m of a query moves only when a tile's maximum exceeds it by more
  // than kLag (log2 units): weights are exp2(s * scale - m) <= 2^kLag (exact in f16's range),
  // and the accumulators are rescaled by exp2(m_old - m_new) only then, so after the first
  // tiles they are rarely touched. Any reference gives the same quotient O / l; the choice
  // depends only on the query's own scores, so it is the same in every grouping of queries.
  // Key 0 is in tile 0 and visible to every query, so m is finite from the first tile on.
  // (S^T of the next tile, from Kn into sn, is computed here too: its matrix products are
  // interleaved with this tile's vector work)
  auto softmax_pv = [&](int kt, f32x16 (&sacc)[2], const char* Vs, const char* Kn, f32x16 (&sn)[2]) {
    if (kt * KT + KT - 1 > wq0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kpos = kt * KT + kb * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (kpos > qpos) sacc[kb][i] = -__builtin_inff();
        }
    }
    scores(Kn, sn);
    float mt = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
    mt = swap_halves_max(mt);
    const float mtile = mt * sl2;
    const float mnew = mtile > m + kLag ? mtile : m;      // (m = -inf on the first tile)
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // exactly 1 when m stays; 0 on the first tile
    // weights, rounded to f16 as the MFMA operand; l adds the rounded weights (v_dot2_f32_f16
    // against ones), the values the products use
    f16x8 pf[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pf[s4][j] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[s4 >> 1][8 * (s4 & 1) + j], sl2, -mnew));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      ps0 = __builtin_amdgcn_fdot2(f16x2{pf[s4][0], pf[s4][1]}, ones, ps0, false);
      ps1 = __builtin_amdgcn_fdot2(f16x2{pf[s4][2], pf[s4][3]}, ones, ps1, false);
      ps0 = __builtin_amdgcn_fdot2(f16x2{pf[s4][4], pf[s4][5]}, ones, ps0, false);
      ps1 = __builtin_amdgcn_fdot2(f16x2{pf[s4][6], pf[s4][7]}, ones, ps1, false);
    }
    const float ps = swap_halves_sum(ps0 + ps1);
    l = l * alpha + ps;
    m = mnew;
    // issue order: each matrix product of the next tile followed by a share of this tile's
    // vector instructions; the K fragment reads run four fragments ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // LDS read
#pragma unroll
    for (int i = 0; i < 2 * NDS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 128 / NDS, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    // accumulators are rescaled only when some lane's reference moved (else alpha = 1)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    }
    // O^T += V^T . P^T over four 16-key steps
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* vr = Vs + va[db] + 16 * s4 * ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vr);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr + 8 * ROWB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const f16x8 vf = __builtin_bit_cast(f16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[s4], o[db], 0, 0, 0);
      }
  };

  // Pipeline. K tile t sits in ks[t % 2], V tile t in vs[t % 2]. Step kt loads K tile kt + 2
  // and V tile kt + 1 into the arrays freed by the barrier that ended the step before, computes
  // S^T of tile kt + 1 (independent of the softmax of tile kt, so the matrix products of one
  // overlap the other's vector work), and finishes tile kt; it ends with a wait for its loads
  // and a barrier. A tile's pool block is read a step before its loads are issued. Every step
  // issues the same loads (a tile past the last is loaded with an empty range: zeros).
  int bv = block_id(0);
  dma(kbase, 0, bv, ks0, true, dk);
  dma(vbase, 0, bv, vs0, true, dv);
  bv = block_id(min(1, n_kt - 1));
  dma(kbase, 1, bv, ks1, 1 < n_kt, dk);
  int bk = block_id(min(2, n_kt - 1));
  __syncthreads();
  f32x16 sa[2], sb[2];
  scores(ks0, sa);
  __syncthreads();  // (step 0 loads K tile 2 into the array just read)
  auto step = [&](int kt, f32x16 (&cur)[2], f32x16 (&nxt)[2], char* kload, const char* kread, char* vload,
                  const char* vread) {
    dma(kbase, kt + 2, bk, kload, kt + 2 < n_kt, dk);
    dma(vbase, kt + 1, bv, vload, kt + 1 < n_kt, dv);
    if (kt < n_kt) {  // (the step past an odd tile count only keeps the loads in step)
      softmax_pv(kt, cur, vread, kread, nxt);  // (S^T past the last tile: zeros, unused)
    }
    // (the scalar load shares a counter with the LDS reads: issued last, it delays none of them)
    bv = bk;
    bk = block_id(min(kt + 3, n_kt - 1));
    __syncthreads();
  };
  // steps in pairs, so that each array's role in a step is fixed
  for (int kt = 0; kt < n_kt; kt += 2) {
    step(kt, sa, sb, ks0, ks1, vs1, vs0);
    step(kt + 1, sb, sa, ks1, ks0, vs0, vs1);
  }

  if (!qvalid) return;
  const float inv = 1.0f / l;
  const int64_t ob = (int64_t)qrow * H * D + (int64_t)head * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g + 4 * hl;
      const float v0 = o[db][4 * g] * inv, v1 = o[db][4 * g + 1] * inv, v2 = o[db][4 * g + 2] * inv,
                  v3 = o[db][4 * g + 3] * inv;
      if constexpr (BF16_OUT) {
        uint2 w;
        w.x = pack_bf16x2(v0, v1);
        w.y = pack_bf16x2(v2, v3);
        *(uint2*)((uint16_t*)a.o + ob + d) = w;
      } else {
        *(float4*)((float*)a.o + ob + d) = make_float4(v0, v1, v2, v3);
      }
    }
}

bool attn_prefill_supported(int head_dim, int group) {
  return (head_dim == 32 || head_dim == 64 || head_dim == 128) && (group == 1 || group == 2);
}

template <int D, int G, int SPLIT>
static hipError_t prefill_launch(const AttnPrefillArgs& a, dim3 g, hipStream_t s) {
  g.y *= SPLIT;
  const dim3 blk(256);
  if (a.out_bf16)
    launch_kernel(attn_prefill_kernel<D, G, SPLIT, true>, g, blk, 0u, s, a);
  else
    launch_kernel(attn_prefill_kernel<D, G, SPLIT, false>, g, blk, 0u, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t prefill_dispatch(const AttnPrefillArgs& a, dim3 g, hipStream_t s) {
  const int group = a.n_heads / a.n_kv_heads;
  if (group == 1) return prefill_launch<D, 1, 1>(a, g, s);
  if (group == 2) return prefill_launch<D, 2, 2>(a, g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s) {
  if (a.b.n_tiles <= 0) return hipSuccess;
  dim3 g(a.n_kv_heads, a.b.n_tiles);  // KV heads fastest: a tile's heads run side by side
  if (a.head_dim == 32) return prefill_dispatch<32>(a, g, s);
  if (a.head_dim == 64) return prefill_dispatch<64>(a, g, s);
  if (a.head_dim == 128) return prefill_dispatch<128>(a, g, s);
  return hipErrorInvalidValue;
}

}  // namespace dec
