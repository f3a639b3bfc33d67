// Seeded sampling of one token per sequence ("Candle model runner", section 2.6 "The sampler
// and PCG32"), in float64 on the device. One workgroup of 1024 threads per sequence:
//
//   1. the sequence's history marks its count table (bit 31: the id occurs in prompt or
//      output; bits 0..30: its occurrences in the output), with integer atomics whose order
//      does not matter; every later read of a logit applies the penalties from that entry
//      (repetition divides a positive value and multiplies any other; an id seen c > 0 times
//      in the output loses frequency * c + presence, two separately rounded operations);
//   2. the largest penalised value (ties to the lowest id) and Z = sum exp(l - max): the
//      logprob of an id is (l - max) - log Z, taken before the temperature;
//   3. temperature 0 returns the largest; otherwise values are divided by T and
//      - top-k: a radix selection (8-bit digits, most significant first) of the k-th largest
//        order-preserving 64-bit key of the tempered value; equal keys at the cut are taken
//        in ascending id order;
//      - with top-p < 1 (then k <= 1024): the k candidates go to LDS in ascending id order,
//        their sum of exp(lt - max) is taken left to right, a bitonic network orders them by
//        (value descending, id ascending) for the nucleus walk, min-p drops those below
//        min_p times the largest probability, and one thread takes the final softmax and the
//        walk over the kept ids left to right in ascending id order;
//      - with top-p = 1: min-p and the final softmax over the whole vocabulary, each thread
//        summing a contiguous range of ids left to right and the ranges combined in order;
//        the walk finds the first id whose cumulative probability exceeds u;
//   4. u takes two outputs of the sequence's PCG32 stream (O'Neill's XSH-RR generator:
//      state' = state * 6364136223846793005 + inc, output = the 32-bit rotation of
//      (old ^ old >> 18) >> 27 by old >> 59): u = ((a >> 5) * 2^26 + (b >> 6)) * 2^-53;
//   5. the history's entries of the count table are set back to zero.
#include "kernels.h"

namespace dec {

namespace {

constexpr int kST = 1024;                     // threads per sequence
constexpr int kNuc = DEC_SAMPLE_MAX_NUCLEUS;  // candidates the nucleus step orders

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

// sum of one value per thread: thread t's value is added after those of threads < t
__device__ double ordered_sum(double v, double* red, double* out) {
  red[threadIdx.x] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int i = 0; i < kST; ++i) s += red[i];
    *out = s;
  }
  __syncthreads();
  const double r = *out;
  __syncthreads();
  return r;
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
  __shared__ int s_i[4];
  __shared__ double s_d[2];
  const int s = blockIdx.x, t = threadIdx.x;
  const SampleSeq q = seqs[s];
  const dec_sampling P = q.p;
  const float* lg = logits + (int64_t)s * ld;
  uint32_t* cnt = cnt_all + (int64_t)s * V;

  // 1. history marks
  for (int i = t; i < q.h.prompt_len; i += kST) {
    const int v = ids[q.h.prompt_offset + i];
    if (v >= 0 && v < V) atomicOr(&cnt[v], 0x80000000u);
  }
  for (int i = t; i < q.h.output_len; i += kST) {
    const int v = ids[q.h.output_offset + i];
    if (v >= 0 && v < V) {
      atomicAdd(&cnt[v], 1u);
      atomicOr(&cnt[v], 0x80000000u);
    }
  }
  __syncthreads();
  auto pen = [&](int v) -> double {
    double l = (double)lg[v];
    const uint32_t c = __hip_atomic_load(&cnt[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c) {
      l = l > 0.0 ? l / P.repetition_penalty : l * P.repetition_penalty;
      const uint32_t n = c & 0x7fffffffu;
      if (n) {
        const double f = P.frequency_penalty * (double)n;
        l -= f + P.presence_penalty;
      }
    }
    return l;
  };

  // 2. the largest value, its lowest id, and Z
  double mx = -__builtin_inf();
  int am = 0x7fffffff;
  for (int v = t; v < V; v += kST) {
    const double l = pen(v);
    if (l > mx) {
      mx = l;
      am = v;
    }
  }
  block_maxarg(mx, am, red, redi);
  // contiguous id range of this thread (sums and walks in ascending id order)
  const int C = (V + kST - 1) / kST, r0 = min(V, t * C), r1 = min(V, r0 + C);
  double zl = 0.0;
  for (int v = r0; v < r1; ++v) zl += exp(pen(v) - mx);
  const double Z = ordered_sum(zl, red, &s_d[0]);
  int tok = am;

  const double T = P.temperature;
  if (T > 0.0) {
    const double mt = mx / T;  // the largest tempered value (division by T > 0 keeps the order)
    auto lt = [&](int v) { return pen(v) / T; };
    const int k = P.top_k;
    const bool use_k = k > 0 && k < V;
    // 3a. top-k: the top `bits` bits of the cut key are pv; krem ids are still to be taken
    // among those whose key starts with pv (all of them unless `ties`)
    uint64_t pv = 0;
    int bits = 0, krem = k;
    bool ties = false;
    if (use_k) {
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        if (t < 256) hist[t] = 0;
        __syncthreads();
        for (int v = t; v < V; v += kST) {
          const uint64_t key = okey(lt(v));
          if (bits == 0 || (key >> (64 - bits)) == pv) atomicAdd(&hist[(key >> shift) & 255u], 1u);
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
    // rank of this thread's first equal key among all equal keys (ties only)
    int eq_base = 0;
    if (ties) {
      int n = 0;
      for (int v = r0; v < r1; ++v) n += okey(lt(v)) == pv;
      redi[t] = n;
      __syncthreads();
      if (t == 0) {
        int a = 0;
        for (int i = 0; i < kST; ++i) {
          const int c = redi[i];
          redi[i] = a;
          a += c;
        }
      }
      __syncthreads();
      eq_base = redi[t];
      __syncthreads();
    }
    // kept by top-k: walks the thread's range in ascending id order (eq counts equal keys seen)
    auto topk_in = [&](uint64_t key, int& eq) -> bool {
      if (!use_k) return true;
      const uint64_t top = key >> (64 - bits);
      if (top > pv) return true;
      if (top < pv) return false;
      if (!ties) return true;
      return eq_base + eq++ < krem;
    };

    if (P.top_p < 1.0) {
      // 3b. nucleus path: the k (<= kNuc) candidates in ascending id order
      int n = 0, eq = 0;
      for (int v = r0; v < r1; ++v) n += topk_in(okey(lt(v)), eq);
      redi[t] = n;
      __syncthreads();
      if (t == 0) {
        int a = 0;
        for (int i = 0; i < kST; ++i) {
          const int c = redi[i];
          redi[i] = a;
          a += c;
        }
        s_i[3] = a;
      }
      __syncthreads();
      int w = redi[t];
      const int nc = s_i[3];
      eq = 0;
      for (int v = r0; v < r1; ++v) {
        const double x = lt(v);
        const uint64_t key = okey(x);
        if (topk_in(key, eq) && w < kNuc) {
          cand_id[w] = v;
          cand_key[w] = key;
          cand_e[w] = exp(x - mt);
          ++w;
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
      if (t == 0) {
        const int m = min(nc, kNuc);
        double zk = 0.0;
        for (int i = 0; i < m; ++i) zk += cand_e[i];
        double c = 0.0;
        for (int j = 0; j < m; ++j) {
          const int i = ord[j];
          c += cand_e[i] / zk;
          keepc[i] = 1;
          if (c >= P.top_p) break;
        }
        if (P.min_p > 0.0) {
          const double qmax = cand_e[ord[0]] / zk;
          for (int i = 0; i < m; ++i)
            if (keepc[i] && cand_e[i] / zk < P.min_p * qmax) keepc[i] = 0;
        }
        double zf = 0.0;
        for (int i = 0; i < m; ++i)
          if (keepc[i]) zf += cand_e[i];
        uint64_t st = rng[2 * s];
        const uint64_t inc = rng[2 * s + 1];
        const uint32_t a = pcg32_next(st, inc), b = pcg32_next(st, inc);
        rng[2 * s] = st;
        const double u = ((double)(a >> 5) * 67108864.0 + (double)(b >> 6)) * (1.0 / 9007199254740992.0);
        int pick = -1;
        c = 0.0;
        for (int i = 0; i < m; ++i) {
          if (!keepc[i]) continue;
          pick = i;
          c += cand_e[i] / zf;
          if (u < c) break;
        }
        s_i[0] = pick >= 0 ? cand_id[pick] : am;
      }
      __syncthreads();
      tok = s_i[0];
      __syncthreads();
    } else {
      // 3c. the whole vocabulary: min-p over the top-k kept ids, then softmax and walk
      double zk = 1.0;
      if (P.min_p > 0.0) {
        double zl2 = 0.0;
        int eq = 0;
        for (int v = r0; v < r1; ++v) {
          const double x = lt(v);
          if (topk_in(okey(x), eq)) zl2 += exp(x - mt);
        }
        zk = ordered_sum(zl2, red, &s_d[0]);
      }
      const double qmax = 1.0 / zk;  // the largest id's probability: exp(0) / zk
      auto kept = [&](double x, double e, int& eq) {
        if (!topk_in(okey(x), eq)) return false;
        return !(P.min_p > 0.0) || e / zk >= P.min_p * qmax;
      };
      double zl3 = 0.0;
      int eq = 0;
      for (int v = r0; v < r1; ++v) {
        const double x = lt(v), e = exp(x - mt);
        if (kept(x, e, eq)) zl3 += e;
      }
      const double zf = ordered_sum(zl3, red, &s_d[0]);
      // the thread's share of the cumulative probability, then the ranges' starting points
      double pl = 0.0;
      int last = -1;
      eq = 0;
      for (int v = r0; v < r1; ++v) {
        const double x = lt(v), e = exp(x - mt);
        if (kept(x, e, eq)) {
          pl += e / zf;
          last = v;
        }
      }
      red[t] = pl;
      redi[t] = last;
      __syncthreads();
      if (t == 0) {
        uint64_t st = rng[2 * s];
        const uint64_t inc = rng[2 * s + 1];
        const uint32_t a = pcg32_next(st, inc), b = pcg32_next(st, inc);
        rng[2 * s] = st;
        s_d[1] = ((double)(a >> 5) * 67108864.0 + (double)(b >> 6)) * (1.0 / 9007199254740992.0);
        double acc = 0.0;
        int lastk = am;
        for (int i = 0; i < kST; ++i) {
          const double c = red[i];
          red[i] = acc;
          acc += c;
          if (redi[i] >= 0) lastk = redi[i];
        }
        s_i[0] = lastk;
      }
      __syncthreads();
      const double u = s_d[1];
      double c = red[t];
      int found = 0x7fffffff;
      eq = 0;
      // (every range walks: its running sum from the range's start may round differently
      // from the start of the next range; the lowest id found wins)
      for (int v = r0; v < r1; ++v) {
        const double x = lt(v), e = exp(x - mt);
        if (kept(x, e, eq)) {
          c += e / zf;
          if (u < c) {
            found = v;
            break;
          }
        }
      }
      const int lastk = s_i[0];
      redi[t] = found;
      __syncthreads();
      for (int sd = kST / 2; sd > 0; sd >>= 1) {
        if (t < sd) redi[t] = min(redi[t], redi[t + sd]);
        __syncthreads();
      }
      tok = redi[0] != 0x7fffffff ? redi[0] : lastk;
      __syncthreads();
    }
  }

  if (t == 0) {
    next[s] = tok;
    if (logprob) logprob[s] = (pen(tok) - mx) - log(Z);
  }
  __syncthreads();
  // 5. leave the count table zero
  for (int i = t; i < q.h.prompt_len; i += kST) {
    const int v = ids[q.h.prompt_offset + i];
    if (v >= 0 && v < V) __hip_atomic_store(&cnt[v], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int i = t; i < q.h.output_len; i += kST) {
    const int v = ids[q.h.output_offset + i];
    if (v >= 0 && v < V) __hip_atomic_store(&cnt[v], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_sample(const float* logits, int64_t ld, int n_seqs, int vocab, const SampleSeq* seqs,
                         const int32_t* ids, uint32_t* counts, uint64_t* rng, int32_t* next, double* logprob,
                         hipStream_t s) {
  if (n_seqs <= 0) return hipSuccess;
  launch_kernel(sample_kernel, dim3(n_seqs), dim3(kST), 0u, s, logits, ld, vocab, seqs, ids, counts, rng, next,
                logprob);
  return hipGetLastError();
}

}  // namespace dec
