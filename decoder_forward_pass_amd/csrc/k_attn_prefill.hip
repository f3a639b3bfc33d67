// Causal grouped-query attention of prefill rows over the paged KV pool, on MFMA
// ("Candle model runner" 2.4, second equation): the flash-style kernel for an f16 pool.
// The other attention paths (rows + combine, decode) are in k_attn.hip.
#include "kernels.h"

namespace dec {

// ---- flash-style prefill attention (f16 pool, MFMA) ----------------------------------------
// Causal attention of one sequence's new rows over its paged keys ("Candle model runner" 2.4,
// second equation; keys up to and including the query's absolute position), read in place from
// the pool. The 128 positions of a query tile are split over SPLIT blocks per KV head (one block
// of 4 G waves, or two blocks of 2 G waves each taking 64 positions; two smaller blocks share a
// CU and run out of step, so one's matrix products overlap the other's softmax and staging);
// wave w takes head w / (4 / SPLIT) of the KV head's group and 32 query positions. The split
// changes no operation applied to a query. Key tiles of 64 positions, aligned to position 0 of
// the sequence, are staged in LDS (K row-major, V transposed, two stages, the next tile loaded
// while the current one is used). Per key tile and wave, with v_mfma_f32_32x32x16_f16:
//   S^T = K . Q^T (keys x queries), scaled into the exp2 domain and causally masked;
//   online softmax per query (a query's 64 scores sit in lanes l and l ^ 32);
//   O^T += V^T . P^T, where P^T is taken from the S^T accumulators as they are: a lane's eight
//   k-slots of k-step s stand for keys 16 s + 8 (j / 4) + 4 (l / 32) + j % 4, a fixed
//   relabelling of the summation index applied to both operands.
// A query sees the key tiles 0 .. floor(pos / 64) in order; a later, fully masked tile leaves
// its state unchanged bit for bit (scale exp2(0) = 1, weights exp2(-inf) = 0, masked values
// zero). The result therefore does not depend on how queries are grouped into tiles, so
// batched, chunked and single-shot prefill agree exactly.

namespace {
constexpr int kPfKT = 64;  // keys per tile
template <int D>
struct PrefillLds {
  static constexpr int KSTR = D + 8;      // K row stride (halves): 32-row fragment reads conflict-free
  // V^T row stride (halves): 34 words, so the 32 rows of a 64-bit fragment read fall on 32
  // distinct bank pairs
  static constexpr int VSTR = kPfKT + 4;
  static constexpr int KS = kPfKT * KSTR, VS = D * VSTR;
  static constexpr size_t bytes = (size_t)2 * (KS + VS) * 2;  // two stages
};
}  // namespace

template <int D, int G, int SPLIT, bool BF16_OUT>
__global__ __launch_bounds__(256 * G / SPLIT) __attribute__((amdgpu_waves_per_eu(SPLIT)))
void attn_prefill_kernel(AttnPrefillArgs a) {
  using L = PrefillLds<D>;
  constexpr int KT = kPfKT, QT = kPrefillQueryTile;
  constexpr int WPH = 4 / SPLIT;           // waves per head
  constexpr int QB = QT / SPLIT;           // query positions per block
  constexpr int NT = 64 * WPH * G;         // threads: G heads x WPH waves of 32 queries
  constexpr int KSTR = L::KSTR, VSTR = L::VSTR;
  constexpr int NDS = D / 16;              // k-steps of S^T over the head dimension
  constexpr int NDB = D / 32;              // 32-row blocks of O^T
  constexpr int NKC = KT * (D / 8);        // 16-byte K chunks per tile
  static_assert(QT == 128 && (SPLIT == 1 || SPLIT == 2), "4 / SPLIT waves of 32 query positions per head");
  extern __shared__ __attribute__((aligned(16))) uint16_t plds[];  // [stage][K | V^T]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int32_t* table = a.b.block_tables + (int64_t)seq * a.b.tbl_stride;
  const int64_t slab = (int64_t)a.n_kv_heads * a.pool.block_tokens * D;
  const uint16_t* kbase = (const uint16_t*)a.pool.base + (int64_t)a.layer * 2 * a.pool.n_blocks * slab +
                          (int64_t)kvh * a.pool.block_tokens * D;
  const uint16_t* vbase = kbase + a.pool.n_blocks * slab;
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

  // ---- staging of key tile kt through registers: K in 16-byte chunks, V in blocks of 2 keys x
  // 8 channels transposed in registers (32 consecutive threads fill one row of V^T). The pool
  // block of every key of a tile is fetched ahead (lane j of each wave: key j of the tile) and
  // handed out by lane shuffles. A key past the context reads the last key's slot (in bounds)
  // and is written to LDS as zeros; nothing is applied to the loaded registers before they are
  // stored, so the loads of a tile stay in flight for a whole step.
  constexpr int KPT = (NKC + NT - 1) / NT;
  constexpr int NV2 = (KT / 2) * (D / 8);  // 2 x 8 V blocks per tile
  constexpr int VPT = (NV2 + NT - 1) / NT;
  const int last_key = ctx_end - 1;
  auto block_ids = [&](int kt) {
    return table[min(kt * KT + lane, last_key) >> bsh];
  };
  struct Regs {
    u32x4 k[KPT], v[VPT][2];
  };
  auto load_tile = [&](int kt, int bids, Regs& r) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int c = min(tid + j * NT, NKC - 1);
      const int key = c / (D / 8), part = c % (D / 8);
      const int kpos = kt * KT + key;
      const int64_t blk = __shfl(bids, key, 64);
      r.k[j] = *(const u32x4*)(kbase + blk * slab + (min(kpos, last_key) & bmask) * D + part * 8);
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vb = min(tid + j * NT, NV2 - 1);
      const int k2 = vb % (KT / 2), d8 = vb / (KT / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int key = k2 * 2 + e, kpos = kt * KT + key;
        const int64_t blk = __shfl(bids, key, 64);
        r.v[j][e] = *(const u32x4*)(vbase + blk * slab + (min(kpos, last_key) & bmask) * D + d8 * 8);
      }
    }
  };
  auto store_tile = [&](int st, int kt, const Regs& r) {
    uint16_t* Ks = plds + (size_t)st * (L::KS + L::VS);
    uint16_t* Vt = Ks + L::KS;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int c = tid + j * NT;
      const int key = c / (D / 8);
      if (NKC % NT == 0 || c < NKC)  // (every thread has KPT chunks when NT divides NKC)
        *(u32x4*)(Ks + key * KSTR + (c % (D / 8)) * 8) = kt * KT + key > last_key ? zero : r.k[j];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int vb = tid + j * NT;
      if (NV2 % NT != 0 && vb >= NV2) continue;
      const int k2 = vb % (KT / 2), d8 = vb / (KT / 2);
      const u32x4 v0 = kt * KT + k2 * 2 > last_key ? zero : r.v[j][0];
      const u32x4 v1 = kt * KT + k2 * 2 + 1 > last_key ? zero : r.v[j][1];
      // v0 / v1 word w holds channels (2w, 2w + 1) of keys 2 k2 / 2 k2 + 1; row d of V^T gets both
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t x0 = v0[d >> 1], x1 = v1[d >> 1];
        *(uint32_t*)(Vt + (d8 * 8 + d) * VSTR + k2 * 2) =
            (d & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
      }
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m = -__builtin_inff(), l = 0.f;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const int n_kt = pmax / KT + 1;

  // Pipeline: tile kt is used from LDS stage kt % 2 while tile kt + 1 (in registers since the
  // previous step) is written to the other stage and tile kt + 2 is requested from memory. The
  // block ids of a tile are requested one step before its data, ahead of the previous tile's
  // loads, so that waiting for them does not wait for those loads. Every step issues the same
  // loads (the last tile is requested again near the end, in bounds and unused), so each wait
  // covers exactly the loads of the step before.
  Regs ra, rb;
  const int b0 = block_ids(0);
  const int b1 = block_ids(min(1, n_kt - 1));
  load_tile(0, b0, ra);
  int ba = block_ids(min(2, n_kt - 1)), bb;
  load_tile(min(1, n_kt - 1), b1, rb);
  store_tile(0, 0, ra);
  __syncthreads();
  auto step = [&](int kt, const Regs& next, Regs& fill, int buse, int& bload) {
    const int st = kt & 1;
    bload = block_ids(min(kt + 3, n_kt - 1));
    load_tile(min(kt + 2, n_kt - 1), buse, fill);
    if (kt < n_kt) {  // (the step past an odd tile count only keeps the loads and stores in step)
    const uint16_t* Ks = plds + (size_t)st * (L::KS + L::VS);
    const uint16_t* Vt = Ks + L::KS;

    // S^T = K . Q^T for the tile's 64 keys (two 32-key blocks)
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NDS; ++ks) {
        const f16x8 kf = __builtin_bit_cast(f16x8, *(const u32x4*)(Ks + (kb * 32 + ql) * KSTR + ks * 16 + hl * 8));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], sacc[kb], 0, 0, 0);
      }
    }
    // online softmax of this lane's query over the tile. Only a tile that reaches past the
    // wave's first query position needs the causal mask; elsewhere every key is visible.
    // The tile maximum is taken over the raw scores and scaled afterwards (scaling by a
    // positive constant is monotone under rounding, so this is the maximum of the scaled
    // scores), and a weight is exp2(s * scale - m) with one rounding. Key 0 is in tile 0 and
    // visible to every query, so m is finite from the first tile on.
    if (kt * KT + KT - 1 > wq0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kpos = kt * KT + kb * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (kpos > qpos) sacc[kb][i] = -__builtin_inff();
        }
    }
    float mt = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mnew = fmaxf(m, mt * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // exp2(-inf) = 0 on the first tile
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], sl2, -mnew));
        sacc[kb][i] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 32, 64);
    l = l * alpha + ps;
    m = mnew;
    // a running maximum that moved in no lane leaves the accumulators as they are (alpha = 1)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    }

    // O^T += V^T . P^T over four 16-key steps
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      f16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = (_Float16)sacc[s4 >> 1][8 * (s4 & 1) + j];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* vr = Vt + (db * 32 + ql) * VSTR + 16 * s4 + 4 * hl;
        const u32x2 lo = *(const u32x2*)vr;
        const u32x2 hi = *(const u32x2*)(vr + 8);
        const f16x8 vf = __builtin_bit_cast(f16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, o[db], 0, 0, 0);
      }
    }
    }
    // (on the last steps this fills the other stage with a tile no wave reads: the stage was
    // last read before the previous barrier, and the loop ends within a step)
    store_tile(st ^ 1, kt + 1, next);
    __syncthreads();
  };
  // steps in pairs, so that the two register sets keep their roles; every step issues the same
  // memory operations, and only the compute of a step past the last tile is skipped
  for (int kt = 0; kt < n_kt; kt += 2) {
    step(kt, rb, ra, ba, bb);
    step(kt + 1, ra, rb, bb, ba);
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
  constexpr size_t lds = PrefillLds<D>::bytes;
  static bool attr = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_prefill_kernel<D, G, SPLIT, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)attn_prefill_kernel<D, G, SPLIT, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  g.y *= SPLIT;
  const dim3 blk(64 * (4 / SPLIT) * G);
  if (a.out_bf16)
    launch_kernel(attn_prefill_kernel<D, G, SPLIT, true>, g, blk, (uint32_t)lds, s, a);
  else
    launch_kernel(attn_prefill_kernel<D, G, SPLIT, false>, g, blk, (uint32_t)lds, s, a);
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
