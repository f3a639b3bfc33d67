// Seeded sampling of one token per sequence ("Candle model runner", section 2.6 "The sampler
// and PCG32"), in float64 on the device. One workgroup of 1024 threads per sequence:
//
//   1. the sequence's history sets one bit per id in LDS (prompt or output) and counts its
//      output occurrences in the sequence's count table (integer atomics: their order does not
//      matter); every pass reads the float32 logits and recomputes an id's penalised value
//      (repetition divides a positive value and multiplies any other; an id seen c > 0 times
//      in the output loses frequency * c + presence, two separately rounded operations), the
//      count table being read for the marked ids only;
//   2. the largest penalised value (ties to the lowest id) and Z = sum exp(l - max): the
//      logprob of an id is (l - max) - log Z, taken before the temperature;
//   3. temperature 0 returns the largest; otherwise values are divided by T and
//      - top-k: a radix selection (8-bit digits, most significant first) of the k-th largest
//        order-preserving 64-bit key of the tempered value; equal keys at the cut are taken
//        in ascending id order;
//      - top-k with k <= 1024 usually avoids the radix passes over the vocabulary: a histogram
//        of the distance below the largest value (buckets of 1/16) bounds the k-th value, the
//        ids above that bound (at most 4096) go to LDS in id order, and the exact top-k is
//        selected among them;
//      - with top-p < 1 and top-k keeping at most 1024 ids, or a top-k selected in LDS: the k
//        candidates sit in LDS in ascending id order, their sum of exp(lt - max) is taken left to right, a
//        bitonic network orders them by (value descending, id ascending) for the nucleus walk,
//        min-p drops those below min_p times the largest probability, and one thread takes
//        the final softmax and the walk over the kept ids left to right in ascending id order;
//      - with top-p < 1 and top-k keeping more than 1024 ids (or none: top_k = 0), the nucleus
//        cut comes from a radix descent by probability mass over the keys (fixed-order digit
//        sums), and the ids it keeps go through the whole-vocabulary path below;
//      - with top-p = 1: e = exp(lt - max) for the ids top-k and min-p keep, 0 for the others
//        (an id whose e underflows to 0 is never drawn); sums over
//        the whole vocabulary reduce each group of 64 consecutive ids by a fixed lane tree and
//        add the groups left to right (one lane per span of groups, then the spans); the walk
//        finds the group where the cumulative probability passes u from those partial sums,
//        then one wave steps id by id;
//   4. u takes two outputs of the sequence's PCG32 stream (O'Neill's XSH-RR generator:
//      state' = state * 6364136223846793005 + inc, output = the 32-bit rotation of
//      (old ^ old >> 18) >> 27 by old >> 59): u = ((a >> 5) * 2^26 + (b >> 6)) * 2^-53;
//   5. the output's entries of the count table are set back to zero.
#include "kernels.h"

namespace dec {

namespace {

constexpr int kST = 1024;                     // threads per sequence
constexpr int kWaves = kST / 64;
constexpr int kNuc = DEC_SAMPLE_MAX_NUCLEUS;  // candidates the nucleus step orders
constexpr int kMaxGroups = 4096;              // groups of 64 ids: vocabularies up to 262,144
constexpr int kU = 8;                         // ids per thread whose loads are issued together
constexpr int kCand = 4096;                   // top-k candidates selected in LDS, at most

// order-preserving key: a larger double has a larger key (finite values and infinities)
__device__ __forceinline__ uint64_t okey(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ uint32_t pcg32_next(uint64_t& state, uint64_t inc) {
  const uint64_t old = state;
  state = old * 6364136223846793005ull + inc;
  const uint32_t xs = (uint32_t)(((old >> 18) ^ old) >> 27);
  const uint32_t rot = (uint32_t)(old >> 59);
  return (xs >> rot) | (xs << ((32u - rot) & 31u));
}

// largest value with the lowest id among equals
__device__ void block_maxarg(double& v, int& id, double* red, int* redi) {
  const int t = threadIdx.x;
  red[t] = v;
  redi[t] = id;
  __syncthreads();
  for (int s = kST / 2; s > 0; s >>= 1) {
    if (t < s) {
      const double ov = red[t + s];
      const int oi = redi[t + s];
      if (ov > red[t] || (ov == red[t] && oi < redi[t])) {
        red[t] = ov;
        redi[t] = oi;
      }
    }
    __syncthreads();
  }
  v = red[0];
  id = redi[0];
  __syncthreads();
}

}  // namespace

__global__ __launch_bounds__(kST) void sample_kernel(const float* __restrict__ logits, int64_t ld, int V,
                                                     const SampleSeq* __restrict__ seqs,
                                                     const int32_t* __restrict__ ids, uint32_t* __restrict__ cnt_all,
                                                     uint64_t* __restrict__ rng, int32_t* __restrict__ next,
                                                     double* __restrict__ logprob) {
#pragma clang fp contract(off)
  __shared__ double red[kST];
  __shared__ int redi[kST];
  __shared__ uint32_t hist[256];
  __shared__ int cand_id[kNuc];
  __shared__ double cand_e[kNuc];
  __shared__ uint64_t cand_key[kNuc];
  __shared__ int ord[kNuc];
  __shared__ uint8_t keepc[kNuc];
  __shared__ double gp[kMaxGroups];           // per group of 64 ids: a partial sum
  __shared__ int gc[kMaxGroups];              // per group: a count, then its exclusive prefix
  __shared__ uint32_t hbits[kMaxGroups * 2];  // one bit per id: in the prompt or the output
  __shared__ double sp[kWaves];               // per span of groups: a partial sum
  __shared__ int cidx[kCand];                 // top-k candidates: ids (keys in gp's storage)
  __shared__ int s_i[4];
  __shared__ double s_d[2];
  const int s = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const SampleSeq q = seqs[s];
  const dec_sampling P = q.p;
  const float* lg = logits + (int64_t)s * ld;
  uint32_t* cnt = cnt_all + (int64_t)s * V;
  const int NG = (V + 63) / 64;                 // groups of 64 consecutive ids
  const int span = (NG + kWaves - 1) / kWaves;  // groups per span (one per wave)
  // Thread t owns the ids v = t (mod kST): in batch i0 the ids i0 + u kST + t, u < kU, whose
  // loads are all issued before any is used; group g = v / 64 is handled by one wave.

  // 1. history: its ids' bits, and the output occurrences in the count table
  for (int i = t; i < NG * 2; i += kST) hbits[i] = 0;
  __syncthreads();
  for (int i = t; i < q.h.prompt_len; i += kST) {
    const int v = ids[q.h.prompt_offset + i];
    if (v >= 0 && v < V) atomicOr(&hbits[v >> 5], 1u << (v & 31));
  }
  for (int i = t; i < q.h.output_len; i += kST) {
    const int v = ids[q.h.output_offset + i];
    if (v >= 0 && v < V) {
      atomicOr(&hbits[v >> 5], 1u << (v & 31));
      atomicAdd(&cnt[v], 1u);
    }
  }
  __syncthreads();
  // the penalised value of id v with logit x (history ids only read the count table)
  auto pen = [&](float x, int v) -> double {
    double l = (double)x;
    if ((hbits[v >> 5] >> (v & 31)) & 1u) {
      l = l > 0.0 ? l / P.repetition_penalty : l * P.repetition_penalty;
      const uint32_t n = __hip_atomic_load(&cnt[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (n) {
        const double f = P.frequency_penalty * (double)n;
        l -= f + P.presence_penalty;
      }
    }
    return l;
  };
  // 2. the largest value (lowest id among equals)
  double mx = -__builtin_inf();
  int am = 0x7fffffff;
  for (int i0 = 0; i0 < V; i0 += kST * kU) {
    float x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = i0 + u * kST + t;
      x[u] = v < V ? lg[v] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = i0 + u * kST + t;
      if (v < V) {
        const double l = pen(x[u], v);
        if (l > mx) {
          mx = l;
          am = v;
        }
      }
    }
  }
  block_maxarg(mx, am, red, redi);

  // Sum of f(x, v) (x: logit of id v; f is called by every lane, v >= V included, and must
  // give 0 there) over the vocabulary in a fixed order: each group of 64 ids by a pairwise
  // lane tree, the groups of a span left to right, the spans left to right.
  auto vocab_sum = [&](auto f) -> double {
    for (int g0 = 0; g0 < NG; g0 += kWaves * kU) {
      float x[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int v = (g0 + u * kWaves) * 64 + t;
        x[u] = v < V ? lg[v] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int g = g0 + u * kWaves + wave;
        const int v = g * 64 + lane;
        double y = f(x[u], v);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) y += __shfl_xor(y, o, 64);
        if (lane == 0 && g < NG) gp[g] = y;
      }
    }
    __syncthreads();
    if (lane == 0) {
      double a = 0.0;
      const int g1 = min(NG, (wave + 1) * span);
#pragma unroll 8
      for (int g = wave * span; g < g1; ++g) a += gp[g];
      sp[wave] = a;
    }
    __syncthreads();
    if (t == 0) {
      double a = 0.0;
      for (int w = 0; w < kWaves; ++w) a += sp[w];
      s_d[0] = a;
    }
    __syncthreads();
    const double r = s_d[0];
    __syncthreads();
    return r;
  };
  // arr[0 .. n) := its exclusive prefix, n <= 4 kST (each thread scans 4 entries, then a
  // doubling scan over the threads); returns the total
  auto prefix4 = [&](int* arr, int n) -> int {
    int loc[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = t * 4 + j;
      loc[j] = g < n ? arr[g] : 0;
      sum += loc[j];
    }
    redi[t] = sum;
    __syncthreads();
    for (int o = 1; o < kST; o <<= 1) {
      const int add = t >= o ? redi[t - o] : 0;
      __syncthreads();
      redi[t] += add;
      __syncthreads();
    }
    int a = redi[t] - sum;  // exclusive
    const int total = redi[kST - 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = t * 4 + j;
      if (g < n) arr[g] = a;
      a += loc[j];
    }
    __syncthreads();
    return total;
  };
  auto group_prefix = [&](int* arr) { return prefix4(arr, NG); };
  const uint64_t lanes_below = lane ? (~0ull >> (64 - lane)) : 0ull;

  const double T = P.temperature;
  const int k = P.top_k;
  const bool use_k = T > 0.0 && k > 0 && k < V;
  const double mt = T > 0.0 ? mx / T : 0.0;  // the largest tempered value (division by T > 0 keeps the order)
  auto lt = [&](float x, int v) { return pen(x, v) / T; };
  auto bucket = [&](double y) { return (mt - y) * 16.0; };  // >= 0; the top-k candidate test of 3a
  // (with a top-k of at most kNuc the Z pass also fills 3a's histogram of bucket(lt))
  const bool hist_in_z = use_k && k <= kNuc;
  if (hist_in_z) {
    if (t < 256) hist[t] = 0;
    __syncthreads();
  }
  const double Z = vocab_sum([&](float x, int v) {
    if (v >= V) return 0.0;
    const double l = pen(x, v);
    if (hist_in_z) {
      const double d = bucket(l / T);
      if (d < 256.0) atomicAdd(&hist[(int)d], 1u);
    }
    return exp(l - mx);
  });
  int tok = am;

  if (T > 0.0) {
    // 3a. top-k with k <= kNuc: candidates first. A histogram of the distance below the largest
    // tempered value, in buckets of 1/16 up to 16 (monotone in the value), gives the bucket b*
    // where the count of larger-or-equal values first reaches k; the ids of buckets <= b* (at
    // most kCand) go to LDS in id order, and the exact top-k by (value descending, id ascending)
    // is selected there into cand_*. Otherwise (more candidates, or k beyond kNuc) the radix
    // selection runs over the whole vocabulary (3a').
    bool lds = hist_in_z;  // the histogram was filled by the Z pass
    int nc = 0;
    uint64_t* ckey = (uint64_t*)gp;
    if (lds) {
      if (t == 0) {
        uint32_t acc = 0;
        int bs = -1;
        for (int b = 0; b < 256; ++b) {
          acc += hist[b];
          if (acc >= (uint32_t)k) {
            bs = b;
            break;
          }
        }
        s_i[0] = bs;
        s_i[1] = (int)acc;
      }
      __syncthreads();
      const int bstar = s_i[0], C = s_i[1];
      __syncthreads();
      lds = bstar >= 0 && C <= kCand;
      if (lds) {
        auto is_cand = [&](double y) {
          const double d = bucket(y);
          return d < 256.0 && (int)d <= bstar;
        };
        for (int g0 = 0; g0 < NG; g0 += kWaves) {
          const int g = g0 + wave;
          const int v = g * 64 + lane;
          const uint64_t m = __ballot(v < V && is_cand(lt(lg[v], v)));
          if (lane == 0 && g < NG) gc[g] = __popcll(m);
        }
        __syncthreads();
        group_prefix(gc);
        for (int g0 = 0; g0 < NG; g0 += kWaves) {
          const int g = g0 + wave;
          const int v = g * 64 + lane;
          const double y = v < V ? lt(lg[v], v) : 0.0;
          const bool in = v < V && is_cand(y);
          const uint64_t m = __ballot(in);
          if (in) {
            const int w = gc[g] + (int)__popcll(m & lanes_below);
            cidx[w] = v;
            ckey[w] = okey(y);
          }
        }
        __syncthreads();
        // the k-th key among the C candidates: radix selection over LDS
        uint64_t cpv = 0;
        int cbits = 0, ckrem = k;
        bool cties = false;
        for (int pass = 0; pass < 8; ++pass) {
          const int shift = 56 - 8 * pass;
          if (t < 256) hist[t] = 0;
          __syncthreads();
          for (int i = t; i < C; i += kST) {
            const uint64_t key = ckey[i];
            if (cbits == 0 || (key >> (64 - cbits)) == cpv) atomicAdd(&hist[(key >> shift) & 255u], 1u);
          }
          __syncthreads();
          if (t == 0) {
            uint32_t acc = 0;
            int sel = 0;
            for (int d = 255; d >= 0; --d) {
              if (acc + hist[d] >= (uint32_t)ckrem) {
                sel = d;
                break;
              }
              acc += hist[d];
            }
            s_i[0] = sel;
            s_i[1] = (int)acc;
            s_i[2] = (int)hist[sel];
          }
          __syncthreads();
          const int sel = s_i[0], above = s_i[1], in_sel = s_i[2];
          __syncthreads();
          ckrem -= above;
          cpv = (cpv << 8) | (uint64_t)sel;
          cbits += 8;
          if (in_sel == ckrem) break;
          cties = pass == 7;
        }
        // equal keys at the cut: their ranks in id order (gc: equal keys before each candidate)
        if (cties) {
          for (int i = t; i < C; i += kST) gc[i] = ckey[i] == cpv;
          __syncthreads();
          prefix4(gc, C);
        }
        // the top-k (exactly k) into cand_* in id order: each thread's 4 consecutive candidates
        int kf[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = t * 4 + j;
          bool in = false;
          if (i < C) {
            const uint64_t top = ckey[i] >> (64 - cbits);
            in = top > cpv || (top == cpv && (!cties || gc[i] < ckrem));
          }
          kf[j] = in;
          sum += in;
        }
        __syncthreads();
        redi[t] = sum;
        __syncthreads();
        for (int o = 1; o < kST; o <<= 1) {
          const int add = t >= o ? redi[t - o] : 0;
          __syncthreads();
          redi[t] += add;
          __syncthreads();
        }
        int w = redi[t] - sum;
        nc = redi[kST - 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = t * 4 + j;
          if (kf[j] && w < kNuc) {
            const uint64_t key = ckey[i];
            const uint64_t b = (key >> 63) ? (key & 0x7fffffffffffffffull) : ~key;  // okey inverted
            cand_id[w] = cidx[i];
            cand_key[w] = key;
            cand_e[w] = exp(__builtin_bit_cast(double, b) - mt);
          }
          w += kf[j];
        }
        __syncthreads();
      }
    }
    // 3a'. top-k over the whole vocabulary: the top `bits` bits of the cut key are pv; krem ids
    // are still to be taken among those whose key starts with pv (all of them unless `ties`)
    uint64_t pv = 0;
    int bits = 0, krem = k;
    bool ties = false;
    if (use_k && !lds) {
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        if (t < 256) hist[t] = 0;
        __syncthreads();
        for (int i0 = 0; i0 < V; i0 += kST * kU) {
          float x[kU];
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int v = i0 + u * kST + t;
            x[u] = v < V ? lg[v] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int v = i0 + u * kST + t;
            if (v < V) {
              const uint64_t key = okey(lt(x[u], v));
              if (bits == 0 || (key >> (64 - bits)) == pv) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
          }
        }
        __syncthreads();
        if (t == 0) {
          uint32_t acc = 0;
          int sel = 0;
          for (int d = 255; d >= 0; --d) {
            if (acc + hist[d] >= (uint32_t)krem) {
              sel = d;
              break;
            }
            acc += hist[d];
          }
          s_i[0] = sel;
          s_i[1] = (int)acc;
          s_i[2] = (int)hist[sel];
        }
        __syncthreads();
        const int sel = s_i[0], above = s_i[1], in_sel = s_i[2];
        __syncthreads();
        krem -= above;
        pv = (pv << 8) | (uint64_t)sel;
        bits += 8;
        if (in_sel == krem) break;
        ties = pass == 7;  // 64 bits and more equal keys than places: the lowest ids are taken
      }
    }
    // equal keys at the cut: their ranks in id order (gc: equal keys before each group)
    if (ties) {
      for (int g0 = 0; g0 < NG; g0 += kWaves) {
        const int g = g0 + wave;
        const int v = g * 64 + lane;
        const uint64_t m = __ballot(v < V && okey(lt(lg[v], v)) == pv);
        if (lane == 0 && g < NG) gc[g] = __popcll(m);
      }
      __syncthreads();
      group_prefix(gc);
    }
    // kept by top-k: tempered value y of lane's id v in group g (called by whole waves: ranks
    // of equal keys at the cut come from a ballot, after those of earlier groups)
    auto kept_tk = [&](int g, int v, double y) -> bool {
      bool in = false, eq = false;
      if (v < V) {
        if (!use_k) {
          in = true;
        } else {
          const uint64_t top = okey(y) >> (64 - bits);
          in = top > pv;
          eq = top == pv;
        }
      }
      if (ties) {
        const uint64_t eqm = __ballot(eq);
        if (eq) in = gc[g] + (int)__popcll(eqm & lanes_below) < krem;
      } else if (eq) {
        in = true;
      }
      return in;
    };

    // a nucleus over more ids than the candidate path orders (top_p < 1 with top-k keeping more
    // than kNuc ids) is cut over the whole vocabulary (3c)
    const bool big_nuc = P.top_p < 1.0 && !lds && (use_k ? k : V) > kNuc;
    if (lds || (P.top_p < 1.0 && !big_nuc)) {
      // 3b. nucleus path over the (<= kNuc) candidates in ascending id order: from 3a, or
      // compacted here from the whole vocabulary (gp's storage holds the per-group counts and
      // their prefix then)
      if (!lds) {
      int* cc = (int*)gp;
      for (int g0 = 0; g0 < NG; g0 += kWaves) {
        const int g = g0 + wave;
        const int v = g * 64 + lane;
        const bool in = kept_tk(g, v, v < V ? lt(lg[v], v) : 0.0);
        const uint64_t m = __ballot(in);
        if (lane == 0 && g < NG) cc[g] = __popcll(m);
      }
      __syncthreads();
      nc = group_prefix(cc);  // (the ties ranks in gc stay as they are)
      for (int g0 = 0; g0 < NG; g0 += kWaves) {
        const int g = g0 + wave;
        const int v = g * 64 + lane;
        const double y = v < V ? lt(lg[v], v) : 0.0;
        const bool in = kept_tk(g, v, y);
        const uint64_t m = __ballot(in);
        if (in) {
          const int w = cc[g] + (int)__popcll(m & lanes_below);
          if (w < kNuc) {
            cand_id[w] = v;
            cand_key[w] = okey(y);
            cand_e[w] = exp(y - mt);
          }
        }
      }
      }
      ord[t] = t < nc ? t : -1;
      keepc[t] = 0;
      __syncthreads();
      // order (value descending, id ascending); empty slots (-1) last
      auto before = [&](int x, int y) {
        if (x < 0) return false;
        if (y < 0) return true;
        return cand_key[x] > cand_key[y] || (cand_key[x] == cand_key[y] && cand_id[x] < cand_id[y]);
      };
      for (int size = 2; size <= kNuc; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          const int j = t ^ stride;
          if (j > t) {
            const int x = ord[t], y = ord[j];
            const bool up = (t & size) == 0;
            if (up ? before(y, x) : before(x, y)) {
              ord[t] = y;
              ord[j] = x;
            }
          }
          __syncthreads();
        }
      }
      // sums left to right in id order by one thread; the divisions by all threads (red holds
      // the quotients), so the sequential walks only add
      const int m = min(nc, kNuc);
      if (t == 0) {
        double z = 0.0;
#pragma unroll 8
        for (int i = 0; i < m; ++i) z += cand_e[i];
        s_d[0] = z;
      }
      __syncthreads();
      const double zk = s_d[0];
      if (t < m) red[t] = cand_e[ord[t]] / zk;  // q of the t-th id in walk order
      __syncthreads();
      if (t == 0) {
        int j = m;  // ids kept by the nucleus: the first j in walk order
        if (P.top_p < 1.0) {
          double c = 0.0;
          for (int i = 0; i < m; ++i) {
            c += red[i];
            if (c >= P.top_p) {
              j = i + 1;
              break;
            }
          }
        }
        s_i[0] = j;
      }
      __syncthreads();
      const double qmax = red[0];
      if (t < s_i[0]) keepc[ord[t]] = 1;
      __syncthreads();
      if (P.min_p > 0.0 && t < m && keepc[t] && cand_e[t] / zk < P.min_p * qmax) keepc[t] = 0;
      __syncthreads();
      if (t == 0) {
        double z = 0.0;
#pragma unroll 8
        for (int i = 0; i < m; ++i)
          if (keepc[i]) z += cand_e[i];
        s_d[0] = z;
      }
      __syncthreads();
      const double zf = s_d[0];
      if (t < m) red[t] = keepc[t] ? cand_e[t] / zf : -1.0;  // the final probabilities; -1: dropped
      __syncthreads();
      if (t == 0) {
        uint64_t st = rng[2 * s];
        const uint64_t inc = rng[2 * s + 1];
        const uint32_t a = pcg32_next(st, inc), b = pcg32_next(st, inc);
        rng[2 * s] = st;
        const double u = ((double)(a >> 5) * 67108864.0 + (double)(b >> 6)) * (1.0 / 9007199254740992.0);
        int pick = -1;
        double c = 0.0;
        for (int i = 0; i < m; ++i) {
          const double pi = red[i];
          if (pi < 0.0) continue;
          pick = i;
          c += pi;
          if (u < c) break;
        }
        s_i[0] = pick >= 0 ? cand_id[pick] : am;
      }
      __syncthreads();
      tok = s_i[0];
      __syncthreads();
    } else {
      // 3c. the whole vocabulary: e = exp(lt - max) for the ids top-k (and, with top-p < 1, the
      // nucleus) keeps, 0 otherwise; min-p over those; softmax and walk
      //
      // The nucleus cut (3c'): walking the top-k ids by (value descending, id ascending), the
      // first id where the cumulative probability reaches top_p is the last one kept. It is found
      // by a radix descent over the order-preserving 64-bit keys of the tempered values (8-bit
      // digits, most significant first): each pass adds the probability of the ids of every digit
      // under the current prefix, and takes the digit where the mass above it plus its own first
      // reaches top_p; the descent ends when that digit holds one id, or after 64 bits with ids of
      // equal value, which are taken in id order until the sum reaches top_p. A digit's mass is
      // a fixed-order sum: within a wave the lanes of one digit are added by a fixed butterfly
      // (digit by digit, lowest lane's digit first) into the wave's histogram held in registers
      // (lane l: digits 4l .. 4l + 3), and the 16 waves' histograms are added in wave order, so
      // the cut is the same on every run; the cumulative probability is the sum of whole digits'
      // masses, equal to the walk's left-to-right sum up to rounding.
      bool nuc_on = false;     // the nucleus predicate is in force (after 3c')
      uint64_t npv = 0;        // the descent's prefix (its top nbits bits of the cut key)
      int nbits = 0, ntake = 0;
      bool nties = false;      // equal keys at the cut: the first ntake in id order are kept
      auto kept_nuc = [&](int g, int v, double y, bool intk) -> bool {  // (whole waves)
        const uint64_t top = okey(y) >> (64 - nbits);
        const bool eq = intk && top == npv;
        bool in = intk && top > npv;
        if (nties) {
          const uint64_t eqm = __ballot(eq);
          if (eq) in = cidx[g] + (int)__popcll(eqm & lanes_below) < ntake;
        } else if (eq) {
          in = true;
        }
        return in;
      };
      auto e_tk = [&](float x, int v, int g) -> double {
        const double y = v < V ? lt(x, v) : 0.0;
        bool in = kept_tk(g, v, y);
        if (nuc_on) in = kept_nuc(g, v, y, in);
        return in ? exp(y - mt) : 0.0;
      };
      double zk = 1.0, qmax = 0.0;
      if (P.min_p > 0.0 || big_nuc) {
        zk = vocab_sum([&](float x, int v) { return e_tk(x, v, v >> 6); });
        qmax = 1.0 / zk;  // the largest id's probability: exp(0) / zk
      }
      if (big_nuc) {
        double above = 0.0;  // probability of the top-k ids above the current prefix's digit
        for (int pass = 0; pass < 8; ++pass) {
          const int shift = 56 - 8 * pass;
          if (t < 256) hist[t] = 0;
          __syncthreads();
          double b0 = 0.0, b1 = 0.0, b2 = 0.0, b3 = 0.0;
          for (int g = wave; g < NG; g += kWaves) {
            const int v = g * 64 + lane;
            const double y = v < V ? lt(lg[v], v) : 0.0;
            const bool intk = kept_tk(g, v, y);
            const uint64_t key = okey(y);
            const bool act = intk && (nbits == 0 || (key >> (64 - nbits)) == npv);
            const int dig = (int)((key >> shift) & 255u);
            if (act) atomicAdd(&hist[dig], 1u);
            const double m = act ? exp(y - mt) / zk : 0.0;
            uint64_t todo = __ballot(act);
            while (todo) {
              const int d = __shfl(dig, __builtin_ctzll(todo), 64);
              const uint64_t mk = __ballot(act && dig == d);
              double x = ((mk >> lane) & 1ull) ? m : 0.0;
#pragma unroll
              for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
              if (lane == (d >> 2)) {
                const int r = d & 3;
                if (r == 0) b0 += x;
                else if (r == 1) b1 += x;
                else if (r == 2) b2 += x;
                else b3 += x;
              }
              todo &= ~mk;
            }
          }
          // the waves' histograms added in wave order: digit 4 l + r into cand_e
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            red[wave * 64 + lane] = r == 0 ? b0 : (r == 1 ? b1 : (r == 2 ? b2 : b3));
            __syncthreads();
            if (t < 64) {
              double a = 0.0;
              for (int w = 0; w < kWaves; ++w) a += red[w * 64 + t];
              cand_e[4 * t + r] = a;
            }
            __syncthreads();
          }
          if (t == 0) {
            double acc = above;
            int sel = -1, last = -1;
            for (int d = 255; d >= 0; --d) {
              if (!hist[d]) continue;
              last = d;
              if (acc + cand_e[d] >= P.top_p) {
                sel = d;
                break;
              }
              acc += cand_e[d];
            }
            if (sel < 0) {  // (rounding kept the total below top_p: every id is kept)
              sel = last;
              acc -= cand_e[last];
            }
            s_i[0] = sel;
            s_i[1] = (int)hist[sel];
            s_d[0] = acc;
          }
          __syncthreads();
          const int sel = s_i[0], cnt = s_i[1];
          above = s_d[0];
          __syncthreads();
          npv = (npv << 8) | (uint64_t)sel;
          nbits += 8;
          if (cnt == 1) break;
          if (pass == 7) {
            // equal values at the cut: each has probability q; in id order they are taken
            // until the walk's sum reaches top_p (their ranks: counts per group, then a ballot)
            if (t == 0) {
              const uint64_t b = (npv >> 63) ? (npv & 0x7fffffffffffffffull) : ~npv;  // okey inverted
              const double qt = exp(__builtin_bit_cast(double, b) - mt) / zk;
              double c = above;
              int j = 0;
              while (j < cnt) {
                c += qt;
                ++j;
                if (c >= P.top_p) break;
              }
              s_i[0] = j;
            }
            for (int g = wave; g < NG; g += kWaves) {
              const int v = g * 64 + lane;
              const double y = v < V ? lt(lg[v], v) : 0.0;
              const bool eq = kept_tk(g, v, y) && okey(y) == npv;
              const uint64_t m = __ballot(eq);
              if (lane == 0) cidx[g] = __popcll(m);
            }
            __syncthreads();
            ntake = s_i[0];
            group_prefix(cidx);
            nties = true;
          }
        }
        nuc_on = true;
      }
      auto e_of = [&](float x, int v) -> double {
        const double e = e_tk(x, v, v >> 6);
        if (P.min_p > 0.0 && !(e / zk >= P.min_p * qmax)) return 0.0;
        return e;
      };
      const double zf = vocab_sum(e_of);
      // group partials of the probabilities (gp), span partials (sp)
      vocab_sum([&](float x, int v) { return e_of(x, v) / zf; });
      if (t == 0) {
        uint64_t st = rng[2 * s];
        const uint64_t inc = rng[2 * s + 1];
        const uint32_t a = pcg32_next(st, inc), b = pcg32_next(st, inc);
        rng[2 * s] = st;
        const double u = ((double)(a >> 5) * 67108864.0 + (double)(b >> 6)) * (1.0 / 9007199254740992.0);
        // the span, then the group, where the cumulative probability passes u
        double acc = 0.0;
        int w = 0;
        for (; w < kWaves - 1; ++w) {
          if (u < acc + sp[w]) break;
          acc += sp[w];
        }
        int g = w * span;
        const int gend = min(NG, (w + 1) * span);
        for (; g < gend - 1; ++g) {
          if (u < acc + gp[g]) break;
          acc += gp[g];
        }
        s_d[1] = u;
        s_d[0] = acc;
        s_i[0] = max(0, g);
      }
      __syncthreads();
      // wave 0 walks id by id from that group on (the id-level running sum decides): each
      // group's probabilities go to LDS and lane 0 adds them in id order
      if (wave == 0) {
        const double u = s_d[1];
        double c = s_d[0];
        int pick = -1, last = -1;
        for (int g = s_i[0]; g < NG && pick < 0; ++g) {
          const int v = g * 64 + lane;
          const double pr = e_of(v < V ? lg[v] : 0.f, v) / zf;
          red[lane] = pr;
          if (lane == 0) {
            for (int j = 0; j < 64 && g * 64 + j < V; ++j) {
              if (!(red[j] > 0.0)) continue;
              last = g * 64 + j;
              c += red[j];
              if (u < c) {
                pick = last;
                break;
              }
            }
          }
          pick = __shfl(pick, 0, 64);
          last = __shfl(last, 0, 64);
          c = __shfl(c, 0, 64);
        }
        // (rounding left u beyond the sum: the last id that can be drawn; else the largest)
        if (lane == 0) s_i[1] = pick >= 0 ? pick : (last >= 0 ? last : am);
      }
      __syncthreads();
      tok = s_i[1];
      __syncthreads();
    }
  }

  if (t == 0) {
    next[s] = tok;
    if (logprob) logprob[s] = (pen(lg[tok], tok) - mx) - log(Z);
  }
  __syncthreads();
  // 5. leave the count table zero
  for (int i = t; i < q.h.output_len; i += kST) {
    const int v = ids[q.h.output_offset + i];
    if (v >= 0 && v < V) __hip_atomic_store(&cnt[v], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_sample(const float* logits, int64_t ld, int n_seqs, int vocab, const SampleSeq* seqs,
                         const int32_t* ids, uint32_t* counts, uint64_t* rng, int32_t* next, double* logprob,
                         hipStream_t s) {
  if (n_seqs <= 0) return hipSuccess;
  if (vocab > kMaxGroups * 64) return hipErrorInvalidValue;
  launch_kernel(sample_kernel, dim3(n_seqs), dim3(kST), 0u, s, logits, ld, vocab, seqs, ids, counts, rng, next,
                logprob);
  return hipGetLastError();
}

}  // namespace dec
