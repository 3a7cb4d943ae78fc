// Token selection for the rows of a step: the argmax, or a draw from the
// row's distribution when sampling is on.
//
// "Break the Sequential Dependency of LLM Inference Using Lookahead
// Decoding" (Summary) states that the method works with sampling as well as
// greedy decoding and leaves the output distribution unchanged, without an
// algorithm.  The reading implemented here:
//   - draw: tokens in order of logit, descending, lower id first on equal
//     logits; keep the first top_k (all when 0); weights
//     exp((z - z_max) / T); keep the shortest prefix holding top_p of the
//     weight; the drawn token is the first kept one whose running weight
//     exceeds u times the kept total;
//   - u for the token at sequence position n: the top 24 bits of word 0 of
//     Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with counter
//     (n low, n high, 0, 0) and the 64-bit seed as key, times 2^-24;
//   - verification is unchanged: a candidate token is accepted when it
//     equals the token selected at its position, so every emitted token is
//     a draw from the model's distribution given the tokens before it, and
//     a lookahead run emits what plain sampled decoding would.
//
// GPU design: one 1024-thread workgroup per row; the row's logits sit in
// LDS (128 KiB, so V <= 32768) and thread t works on tokens t + 1024 i.  The order is
// a 64-bit key per token: order-preserving bits of the fp32 logit, then the
// complemented token id, so keys are distinct and "earlier in the order" is
// "larger key".  A selection (the k-th key, or the key where the running
// weight from the top passes a target) descends 4 bits at a time: per
// level every thread bins its live tokens by the next digit (16 weight and
// 16 count sums), a fixed-order block reduction gives the totals and every
// thread takes the same digit; it stops when one token is left.  Sums run
// in a fixed order, so a row's decision is the same on every run.
#include "la_epilogue.h"

namespace la {

namespace {

constexpr int SEL_T = 1024;            // threads per row
constexpr int SEL_PER = SAMPLE_MAX_VOCAB / SEL_T;
constexpr int SEL_WAVES = SEL_T / 64;

struct SelShared {
  float w[SEL_WAVES][16];
  uint32_t c[SEL_WAVES][16];
  float wt[16];
  uint32_t ct[16];
  float f[SEL_WAVES];
  int32_t i[SEL_WAVES];
  unsigned long long key;
};

// Philox4x32-10: word 0 of the output block.
__device__ inline uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                        uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    const uint32_t lo0 = c0 * 0xD2511F53u, hi0 = __umulhi(c0, 0xD2511F53u);
    const uint32_t lo1 = c2 * 0xCD9E8D57u, hi1 = __umulhi(c2, 0xCD9E8D57u);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

__device__ inline float uniform_at(uint32_t seed_lo, uint32_t seed_hi, long long pos) {
  const unsigned long long p = (unsigned long long)pos;
  const uint32_t w = philox_word0((uint32_t)p, (uint32_t)(p >> 32), 0u, 0u, seed_lo, seed_hi);
  return (float)(w >> 8) * (1.0f / 16777216.0f);
}

// Order key: larger = earlier in the draw order.
__device__ inline unsigned long long order_key(float z, int j) {
  uint32_t b = __float_as_uint(z);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)b << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ inline float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline uint32_t wave_sum_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over the block in a fixed order (wave trees, then waves in order).
__device__ inline float block_sum(float v, SelShared& sh) {
  v = wave_sum_f(v);
  if ((threadIdx.x & 63) == 0) sh.f[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int q = 0; q < SEL_WAVES; q++) t += sh.f[q];
  __syncthreads();
  return t;
}

// Largest logit, lowest id on ties, over the block.
__device__ inline void block_argmax(float& bv, int& bi, SelShared& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if ((threadIdx.x & 63) == 0) {
    sh.f[threadIdx.x >> 6] = bv;
    sh.i[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  bv = sh.f[0];
  bi = sh.i[0];
  for (int q = 1; q < SEL_WAVES; q++)
    if (sh.f[q] > bv || (sh.f[q] == bv && sh.i[q] < bi)) {
      bv = sh.f[q];
      bi = sh.i[q];
    }
  __syncthreads();
}

// Walk the live tokens (key >= lo) from the largest key down and return
// the key of the token where the running total first reaches the target:
// by count (weighted false: the kth token, kth >= 1), or by weight
// (running weight >= target, or > target when strict).  If rounding leaves
// no digit that reaches it, the walk takes the last live digit.
__device__ unsigned long long descend(const float* zl, float zmax, float invT, int V,
                                      unsigned long long lo, bool weighted, uint32_t kth,
                                      float target, bool strict, SelShared& sh) {
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  unsigned long long prefix = 0ull, mask = 0ull;
  float acc = 0.f;
  uint32_t cacc = 0;
  for (int shift = 60; shift >= 0; shift -= 4) {
    float hw[16];
    uint32_t hc[16];
#pragma unroll
    for (int d = 0; d < 16; d++) {
      hw[d] = 0.f;
      hc[d] = 0u;
    }
#pragma unroll 2
    for (int e = 0; e < SEL_PER; e++) {
      const int j = tid + e * SEL_T;
      if (j >= V) break;
      const float ze = zl[j];
      const unsigned long long K = order_key(ze, j);
      if (K < lo || (K & mask) != prefix) continue;
      const int dg = (int)((K >> shift) & 15ull);
      const float we = weighted ? expf((ze - zmax) * invT) : 0.f;
#pragma unroll
      for (int d = 0; d < 16; d++) {
        hw[d] += dg == d ? we : 0.f;
        hc[d] += dg == d ? 1u : 0u;
      }
    }
#pragma unroll
    for (int d = 0; d < 16; d++) {
      hw[d] = wave_sum_f(hw[d]);
      hc[d] = wave_sum_u(hc[d]);
    }
    if (ln == 0) {
#pragma unroll
      for (int d = 0; d < 16; d++) {
        sh.w[wv][d] = hw[d];
        sh.c[wv][d] = hc[d];
      }
    }
    __syncthreads();
    if (tid < 16) {
      float s = 0.f;
      uint32_t c = 0u;
      for (int q = 0; q < SEL_WAVES; q++) {
        s += sh.w[q][tid];
        c += sh.c[q][tid];
      }
      sh.wt[tid] = s;
      sh.ct[tid] = c;
    }
    __syncthreads();
    // every thread takes the same digit from the same totals
    int pick = -1, last = -1;
    {
      float a = acc;
      uint32_t ca = cacc;
      for (int d = 15; d >= 0; d--) {
        const uint32_t c = sh.ct[d];
        if (c == 0u) continue;
        last = d;
        const bool hit = weighted ? (strict ? a + sh.wt[d] > target : a + sh.wt[d] >= target)
                                  : ca + c >= kth;
        if (hit) {
          pick = d;
          break;
        }
        a += sh.wt[d];
        ca += c;
      }
    }
    if (pick < 0) pick = last < 0 ? 0 : last;  // (no live token cannot happen)
    for (int d = 15; d > pick; d--) {
      acc += sh.wt[d];
      cacc += sh.ct[d];
    }
    const bool single = sh.ct[pick] == 1u;
    prefix |= (unsigned long long)pick << shift;
    mask |= 15ull << shift;
    __syncthreads();  // the totals are rewritten by the next level
    if (single) {
      for (int e = 0; e < SEL_PER; e++) {
        const int j = tid + e * SEL_T;
        if (j >= V) break;
        const unsigned long long K = order_key(zl[j], j);
        if (K >= lo && (K & mask) == prefix) sh.key = K;
      }
      __syncthreads();
      const unsigned long long k = sh.key;
      __syncthreads();
      return k;
    }
  }
  return prefix;
}

// The row's argmax (lowest id on ties) from its copy in LDS.
__device__ inline int row_argmax(const float* zl, int V, float* vmax, SelShared& sh) {
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int j = threadIdx.x; j < V; j += SEL_T) {
    const float v = zl[j];
    if (v > bv) {  // j ascends: the first of equal values stays
      bv = v;
      bi = j;
    }
  }
  block_argmax(bv, bi, sh);
  if (vmax) *vmax = bv;
  return bi;
}

// One row's draw; zl holds the row in LDS.
__device__ int draw_row(const float* zl, int V, const SampleParams& p, float u, SelShared& sh) {
  const int tid = threadIdx.x;
  float zmax;
  row_argmax(zl, V, &zmax, sh);
  const float invT = 1.f / p.temperature;  // weights exp((z - zmax) * invT), recomputed
  unsigned long long lo = 0ull;
  if (p.top_k > 0 && p.top_k < V)
    lo = descend(zl, zmax, invT, V, 0ull, false, (uint32_t)p.top_k, 0.f, false, sh);
  auto kept_sum = [&](unsigned long long lo_key) {
    float s = 0.f;
    for (int j = tid; j < V; j += SEL_T) {
      const float ze = zl[j];
      if (order_key(ze, j) >= lo_key) s += expf((ze - zmax) * invT);
    }
    return block_sum(s, sh);
  };
  if (p.top_p < 1.f) {
    const float zk = kept_sum(lo);
    lo = descend(zl, zmax, invT, V, lo, true, 0u, p.top_p * zk, false, sh);
  }
  const float zs = kept_sum(lo);
  const unsigned long long ks = descend(zl, zmax, invT, V, lo, true, 0u, u * zs, true, sh);
  return (int)(0xFFFFFFFFu - (uint32_t)(ks & 0xFFFFFFFFull));
}

// Copy a row of logits to LDS (and wait for every thread's part).
__device__ inline void load_row(const float* __restrict__ row, int V, float* zl) {
  for (int j = threadIdx.x; j < V; j += SEL_T) zl[j] = row[j];
  __syncthreads();
}

__global__ __launch_bounds__(SEL_T) void k_select(const float* __restrict__ logits, int V, int M,
                                                  int T, int mode, int W, int N,
                                                  const DevState* __restrict__ st,
                                                  const int32_t* __restrict__ relpos,
                                                  const SampleParams* __restrict__ sp,
                                                  int32_t* __restrict__ out) {
  __shared__ SelShared sh;
  __shared__ float zl[SAMPLE_MAX_VOCAB];
  const int r = blockIdx.x;
  int b = 0;
  bool draw;
  if (mode == MODE_STEP) {
    b = r / T;
    const RowDesc rd = row_desc(r - b * T, W, N);
    draw = rd.kind == 0 || (rd.kind == 2 && rd.a < st[b].n_cand);
  } else {
    draw = r == M - 1;
  }
  const SampleParams p = sp[b];
  draw = draw && p.temperature > 0.f;  // uniform over the workgroup
  load_row(logits + (size_t)r * V, V, zl);
  int tok;
  if (draw) {
    const long long pos = (long long)st[b].L + relpos[r] + 1;
    tok = draw_row(zl, V, p, uniform_at(p.seed_lo, p.seed_hi, pos), sh);
  } else {
    tok = row_argmax(zl, V, nullptr, sh);
  }
  if (threadIdx.x == 0) out[r] = tok;
}

__global__ __launch_bounds__(SEL_T) void k_sample_rows(const float* __restrict__ logits, int V,
                                                       SampleParams p,
                                                       const int64_t* __restrict__ positions,
                                                       int32_t* __restrict__ out) {
  __shared__ SelShared sh;
  __shared__ float zl[SAMPLE_MAX_VOCAB];
  const int r = blockIdx.x;
  load_row(logits + (size_t)r * V, V, zl);
  const int tok = draw_row(zl, V, p, uniform_at(p.seed_lo, p.seed_hi, positions[r]), sh);
  if (threadIdx.x == 0) out[r] = tok;
}

}  // namespace

void launch_select(const float* logits, int M, int V, int T, int mode, int W, int N,
                   const DevState* st, const int32_t* relpos, const SampleParams* sp,
                   int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_select, dim3(M), dim3(SEL_T), 0, s, logits, V, M, T, mode, W, N, st, relpos,
                     sp, out);
}

void launch_sample_rows(const float* logits, int rows, int V, const SampleParams& p,
                        const int64_t* positions, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_sample_rows, dim3(rows), dim3(SEL_T), 0, s, logits, V, p, positions, out);
}

}  // namespace la
