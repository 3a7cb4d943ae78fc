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
// GPU design: one 1024-thread workgroup per row; thread t keeps, for the
// tokens j = t + 1024 i (i < 32, so V <= 32768), the order key of the logit
// (order-preserving bits of the fp32 value) and its weight in registers.
// The draw order is by key, descending, then by token id, ascending.  A
// selection (the k-th token in that order, or the token where the running
// weight first reaches or exceeds a target) is a bitwise search for the
// largest key whose running total (over tokens with key >= it) still meets
// the target: one pass over the registers and one fixed-order block sum
// per bit; equal keys are then told apart by a search over token ids.  Sums
// run in a fixed order, so a row's decision is the same on every run.
#include "la_epilogue.h"

namespace la {

namespace {

constexpr int SEL_T = 1024;  // threads per row
constexpr int SEL_PER = SAMPLE_MAX_VOCAB / SEL_T;
constexpr int SEL_WAVES = SEL_T / 64;

constexpr int SEL_KEPT = 64;  // top-k up to this: top-p and the draw on the kept tokens

struct SelShared {
  float f[2][SEL_WAVES];  // double-buffered: one barrier per block sum
  uint32_t n[2][SEL_WAVES];
  int32_t i[SEL_WAVES];
  int32_t tok;
  uint32_t cnt;                // kept tokens appended
  uint32_t kkey[SEL_KEPT];     // their order keys, ids and weights (append order)
  int32_t kid[SEL_KEPT];
  float kw[SEL_KEPT];
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

// Order key of a finite logit: larger logit, larger key (never 0).
__device__ inline uint32_t order_key(float z) {
  const uint32_t b = __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Sum over a wave in a fixed order with DPP lane moves (VALU, no LDS round
// trip): within quads (quad_perm [1,0,3,2], [2,3,0,1]), then within rows of
// 16 (row_ror 4, 8), so every lane holds its row's sum; the four row sums
// are read from lanes 0, 16, 32, 48 and added in order.
__device__ inline uint32_t row_sum_u(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
  return v;
}
__device__ inline float row_sum_f(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  return v;
}
__device__ inline float wave_sum_f(float v) {
  v = row_sum_f(v);
  return ((__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32))) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
}
__device__ inline uint32_t wave_sum_u(uint32_t v) {
  v = row_sum_u(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// (weight, count) summed over the block in a fixed order; buf alternates
// between calls so one barrier suffices.
struct Pair {
  float s;
  uint32_t n;
};
__device__ inline Pair block_pair(float s, uint32_t n, SelShared& sh, int& buf) {
  s = wave_sum_f(s);
  n = wave_sum_u(n);
  if ((threadIdx.x & 63) == 0) {
    sh.f[buf][threadIdx.x >> 6] = s;
    sh.n[buf][threadIdx.x >> 6] = n;
  }
  __syncthreads();
  Pair p{0.f, 0u};
  for (int q = 0; q < SEL_WAVES; q++) {
    p.s += sh.f[buf][q];
    p.n += sh.n[buf][q];
  }
  buf ^= 1;
  return p;
}

// Count only (the count-based selections carry no weights).
__device__ inline uint32_t block_count(uint32_t n, SelShared& sh, int& buf) {
  n = wave_sum_u(n);
  if ((threadIdx.x & 63) == 0) sh.n[buf][threadIdx.x >> 6] = n;
  __syncthreads();
  uint32_t t = 0u;
  for (int q = 0; q < SEL_WAVES; q++) t += sh.n[buf][q];
  buf ^= 1;
  return t;
}
__device__ inline Pair block_total(bool weighted, float s, uint32_t n, SelShared& sh, int& buf) {
  if (weighted) return block_pair(s, n, sh, buf);
  return Pair{0.f, block_count(n, sh, buf)};
}

// Largest logit, lowest id on ties, over the block.
__device__ inline int block_argmax(const float (&z)[SEL_PER], int V, float* vmax, SelShared& sh) {
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int e = 0; e < SEL_PER; e++) {
    const int j = threadIdx.x + e * SEL_T;
    if (j < V && z[e] > bv) {  // j ascends per thread: the first of equal values stays
      bv = z[e];
      bi = j;
    }
  }
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
    sh.f[0][threadIdx.x >> 6] = bv;
    sh.i[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  bv = sh.f[0][0];
  bi = sh.i[0];
  for (int q = 1; q < SEL_WAVES; q++)
    if (sh.f[0][q] > bv || (sh.f[0][q] == bv && sh.i[q] < bi)) {
      bv = sh.f[0][q];
      bi = sh.i[q];
    }
  __syncthreads();
  if (vmax) *vmax = bv;
  return bi;
}

// Tokens out of play carry key 0 (a real key is never 0).  A selection
// returns (key, token) of the token in the draw order where the running
// total over the tokens in play first meets the target: by count
// (WEIGHTED false: the kth token) or by weight (>= target, or > target
// when strict).  Rounding that leaves no such token gives the last token
// in play.
struct KeyTok {
  uint32_t key;
  int tok;
};
template <bool WEIGHTED>
__device__ KeyTok select_token(const uint32_t (&k)[SEL_PER], const float (&w)[SEL_PER],
                               uint32_t kth, float target, bool strict, SelShared& sh,
                               int& buf) {
  const int tid = threadIdx.x;
  auto meets = [&](float s, uint32_t n) {
    return WEIGHTED ? (strict ? s > target : s >= target) : n >= kth;
  };
  // running total of the tokens with key >= c (weights, or counts)
  auto total_ge = [&](uint32_t c) {
    float s = 0.f;
    uint32_t n = 0u;
#pragma unroll
    for (int e = 0; e < SEL_PER; e++) {
      if (WEIGHTED) s += k[e] >= c ? w[e] : 0.f;
      else n += k[e] >= c ? 1u : 0u;
    }
    return block_total(WEIGHTED, s, n, sh, buf);
  };
  // the largest key t whose running total meets the target
  uint32_t t = 0u;
  for (int bit = 31; bit >= 0; bit--) {
    const uint32_t c = t | (1u << bit);
    const Pair p = total_ge(c);
    if (meets(p.s, p.n)) t = c;
  }
  // the tokens at t (equal logits) go in id order
  uint32_t ne = 0u;
#pragma unroll
  for (int e = 0; e < SEL_PER; e++) ne += (t != 0u && k[e] == t) ? 1u : 0u;
  const uint32_t neq = block_count(ne, sh, buf);
  if (neq <= 1u) {
    // one token at t; or none (rounding): the last token in play, i.e. the
    // smallest key, highest id among equals
    if (neq == 0u) {
      uint32_t mk = 0xFFFFFFFFu;
#pragma unroll
      for (int e = 0; e < SEL_PER; e++)
        if (k[e] != 0u) mk = min(mk, k[e]);
      for (int o = 32; o > 0; o >>= 1) mk = min(mk, (uint32_t)__shfl_xor((int)mk, o));
      if ((tid & 63) == 0) sh.n[buf][tid >> 6] = mk;
      __syncthreads();
      t = 0xFFFFFFFFu;
      for (int q = 0; q < SEL_WAVES; q++) t = min(t, sh.n[buf][q]);
      buf ^= 1;
    }
    int hi = -1;
#pragma unroll
    for (int e = 0; e < SEL_PER; e++)
      if (k[e] == t) hi = tid + e * SEL_T;
    for (int o = 32; o > 0; o >>= 1) hi = max(hi, __shfl_xor(hi, o));
    if ((tid & 63) == 0) sh.i[tid >> 6] = hi;
    __syncthreads();
    int tok = -1;
    for (int q = 0; q < SEL_WAVES; q++) tok = max(tok, sh.i[q]);
    __syncthreads();
    return KeyTok{t, tok};
  }
  // several tokens at t: the smallest id J with (total above t) + (their
  // total up to J) meeting the target
  const Pair above = t == 0xFFFFFFFFu ? Pair{0.f, 0u} : total_ge(t + 1u);
  int J = 0;
  for (int bit = 14; bit >= 0; bit--) {
    const int c = J + (1 << bit) - 1;  // test ids <= c
    float s = 0.f;
    uint32_t n = 0u;
#pragma unroll
    for (int e = 0; e < SEL_PER; e++) {
      const bool in = k[e] == t && tid + e * SEL_T <= c;
      s += in ? w[e] : 0.f;
      n += in ? 1u : 0u;
    }
    const Pair p = block_total(WEIGHTED, s, n, sh, buf);
    if (!meets(above.s + p.s, above.n + p.n)) J += 1 << bit;
  }
  return KeyTok{t, J};
}

// Take the tokens after (key, tok) in the draw order out of play.
__device__ inline void cut_after(uint32_t (&k)[SEL_PER], const KeyTok& kt) {
#pragma unroll
  for (int e = 0; e < SEL_PER; e++) {
    const int j = threadIdx.x + e * SEL_T;
    if (k[e] < kt.key || (k[e] == kt.key && j > kt.tok)) k[e] = 0u;
  }
}

// Top-p and the draw over at most SEL_KEPT kept tokens (the rest out of
// play), by wave 0: the kept tokens are gathered in LDS, sorted into the
// draw order (key descending, id ascending: a total order, so the result
// does not depend on the gather order), and their weights summed in that
// order; the same selections as select_token on the same weights, with the
// running totals summed token by token in the draw order.
__device__ int draw_kept(const uint32_t (&k)[SEL_PER], const float (&w)[SEL_PER], float top_p,
                         float u, SelShared& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.cnt = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < SEL_PER; e++)
    if (k[e] != 0u) {
      const uint32_t at = atomicAdd(&sh.cnt, 1u);
      if (at < SEL_KEPT) {  // the count-exact top-k cut keeps exactly top_k <= SEL_KEPT
        sh.kkey[at] = k[e];
        sh.kid[at] = tid + e * SEL_T;
        sh.kw[at] = w[e];
      }
    }
  __syncthreads();
  if (tid < 64) {
    const uint32_t n = min(sh.cnt, (uint32_t)SEL_KEPT);
    uint32_t key = tid < (int)n ? sh.kkey[tid] : 0u;  // padding sorts last
    int id = tid < (int)n ? sh.kid[tid] : 0x7fffffff;
    float wt = tid < (int)n ? sh.kw[tid] : 0.f;
    // bitonic sort over the wave into the draw order
    for (int kk = 2; kk <= 64; kk <<= 1)
      for (int j = kk >> 1; j > 0; j >>= 1) {
        const uint32_t pkey = (uint32_t)__shfl_xor((int)key, j);
        const int pid = __shfl_xor(id, j);
        const float pw = __shfl_xor(wt, j);
        const bool self_first = key > pkey || (key == pkey && id < pid);
        const bool lower = (tid & j) == 0, up = (tid & kk) == 0;
        if (self_first != (lower == up)) {
          key = pkey;
          id = pid;
          wt = pw;
        }
      }
    // running totals in the draw order, token by token
    float run = 0.f, mine = 0.f;
    for (int q = 0; q < 64; q++) {
      run += __shfl(wt, q);
      if (q == tid) mine = run;
    }
    const float total = __shfl(mine, (int)n - 1);
    int last = (int)n - 1;  // last kept token
    if (top_p < 1.f) {
      const uint64_t m = __ballot(tid < (int)n && mine >= top_p * total);
      if (m) last = __ffsll((unsigned long long)m) - 1;
    }
    const float kept = __shfl(mine, last);
    const uint64_t m = __ballot(tid <= last && mine > u * kept);
    const int at = m ? __ffsll((unsigned long long)m) - 1 : last;
    const int tok = __shfl(id, at);
    if (tid == 0) sh.tok = tok;
  }
  __syncthreads();
  const int tok = sh.tok;
  __syncthreads();
  return tok;
}

// One row's draw; z holds the thread's logits (tokens past V unused).
__device__ int draw_row(const float (&z)[SEL_PER], int V, const SampleParams& p, float u,
                        SelShared& sh) {
  float zmax;
  block_argmax(z, V, &zmax, sh);
  const float invT = 1.f / p.temperature;
  uint32_t k[SEL_PER];
  float w[SEL_PER];
#pragma unroll
  for (int e = 0; e < SEL_PER; e++) {
    const int j = threadIdx.x + e * SEL_T;
    k[e] = j < V ? order_key(z[e]) : 0u;
    w[e] = j < V ? expf((z[e] - zmax) * invT) : 0.f;
  }
  int buf = 0;
  if (p.top_k > 0 && p.top_k < V) {
    cut_after(k, select_token<false>(k, w, (uint32_t)p.top_k, 0.f, false, sh, buf));
    if (p.top_k <= SEL_KEPT) return draw_kept(k, w, p.top_p, u, sh);
  }
  auto total = [&]() {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < SEL_PER; e++) s += k[e] != 0u ? w[e] : 0.f;
    return block_pair(s, 0u, sh, buf).s;
  };
  if (p.top_p < 1.f) {
    const float zk = total();
    cut_after(k, select_token<true>(k, w, 0u, p.top_p * zk, false, sh, buf));
  }
  const float zs = total();
  return select_token<true>(k, w, 0u, u * zs, true, sh, buf).tok;
}

__device__ inline void load_row(const float* __restrict__ row, int V, float (&z)[SEL_PER]) {
#pragma unroll
  for (int e = 0; e < SEL_PER; e++) {
    const int j = threadIdx.x + e * SEL_T;
    z[e] = j < V ? row[j] : -INFINITY;
  }
}

__global__ __launch_bounds__(SEL_T) void k_select(const float* __restrict__ logits, int V, int M,
                                                  int T, int mode, int W, int N,
                                                  const DevState* __restrict__ st,
                                                  const int32_t* __restrict__ relpos,
                                                  const SampleParams* __restrict__ sp,
                                                  int32_t* __restrict__ out) {
  __shared__ SelShared sh;
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
  float z[SEL_PER];
  load_row(logits + (size_t)r * V, V, z);
  int tok;
  if (draw) {
    const long long pos = (long long)st[b].L + relpos[r] + 1;
    tok = draw_row(z, V, p, uniform_at(p.seed_lo, p.seed_hi, pos), sh);
  } else {
    tok = block_argmax(z, V, nullptr, sh);
  }
  if (threadIdx.x == 0) out[r] = tok;
}

__global__ __launch_bounds__(SEL_T) void k_sample_rows(const float* __restrict__ logits, int V,
                                                       SampleParams p,
                                                       const int64_t* __restrict__ positions,
                                                       int32_t* __restrict__ out) {
  __shared__ SelShared sh;
  const int r = blockIdx.x;
  float z[SEL_PER];
  load_row(logits + (size_t)r * V, V, z);
  const int tok = draw_row(z, V, p, uniform_at(p.seed_lo, p.seed_hi, positions[r]), sh);
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
