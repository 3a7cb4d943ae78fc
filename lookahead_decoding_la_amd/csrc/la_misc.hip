// Small kernels of the lookahead step: block assembly + embedding gather,
// RMSNorm, greedy verification with window shift and n-gram pool update, KV
// compaction, and fills.  (Per-row token selection: la_sample.hip.)
//
// Method: "Break the Sequential Dependency of LLM Inference Using Lookahead
// Decoding", summary page, Summary and Key points ("Tuning knobs").  Here:
// the window's column diagonals become new n-grams stored per lead token
// (at most G each), the stored n-grams that start with the current token are
// verified inside the step's own forward pass, and the longest agreeing prefix is
// emitted, so the output is that of plain decoding.
#include "la_epilogue.h"

namespace la {

// ---------------------------------------------------------------------------

__global__ void k_fill_u32(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

void launch_fill_u32(void* p, uint32_t v, size_t n, hipStream_t s) {
  if (!n) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, v, n);
}

// ---------------------------------------------------------------------------
// Block assembly: row r's token and relative position, then its embedding.
//   step mode: row 0 = current token; window row (l, j) = win[l-1][j];
//   candidate row (g, i) = i-th token of the g-th pool entry of the current
//   token (oldest entry first), or token 0 for an empty slot (such rows are
//   isolated by the mask and never committed);
//   causal mode: row r = prompt[r] at relative position r.
// In step mode row r is block row r % T of sequence r / T, which has its own
// state, window and pool.

__global__ void k_assemble(int mode, const DevState* __restrict__ st,
                           const int32_t* __restrict__ win, const int32_t* __restrict__ pool_len,
                           const int32_t* __restrict__ pool, const int32_t* __restrict__ prompt,
                           int T, int V, int W, int N, int G, int32_t* tokens, int32_t* relpos,
                           DevState* st_w, const void* __restrict__ emb, int d, int bf16,
                           float* __restrict__ x, const uint16_t* __restrict__ nw, float eps,
                           uint16_t* __restrict__ xnf, int MTT, float* __restrict__ ssq,
                           const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
                           float* __restrict__ rope_rows) {
  __shared__ float sh[4];
  const int r = blockIdx.x;
  int tok, rp;
  const DevState* sr = st;  // the row's sequence
  if (mode == MODE_STEP) {
    const int b = r / T, rl = r - b * T;
    sr = st + b;
    const int32_t* wb = win + (size_t)b * (N - 1) * W;
    const int32_t* pb = pool + (size_t)b * V * G * (N - 1);
    const int cur = sr->cur;
    int nc = G > 0 ? pool_len[(size_t)b * V + cur] : 0;
    nc = nc < G ? nc : G;
    const RowDesc rd = row_desc(rl, W, N);
    rp = row_relpos(rd);
    if (rd.kind == 0) tok = cur;
    else if (rd.kind == 1) tok = wb[(rd.a - 1) * W + rd.b];
    else tok = rd.a < nc ? pb[((size_t)cur * G + rd.a) * (N - 1) + (rd.b - 1)] : 0;
    if (rl == 0 && threadIdx.x == 0) st_w[b].n_cand = nc;
  } else {
    tok = prompt[r];
    rp = r;
  }
  if (threadIdx.x == 0) {
    tokens[r] = tok;
    relpos[r] = rp;
  }
  float* xr = x + (size_t)r * d;
  if (bf16) {
    // this row's rotary factors (head_dim 128: 64 pairs), gathered once per
    // block for every layer's QKV reduce
    if (threadIdx.x < 128) {
      const size_t pos = (size_t)(sr->L + rp);
      const int i = threadIdx.x & 63;
      rope_rows[r * 128 + threadIdx.x] =
          threadIdx.x < 64 ? rope_cos[pos * 64 + i] : rope_sin[pos * 64 + i];
    }
    // 8 columns per thread per pass (d % 128 == 0 for the bf16 kernels,
    // d <= 8192: at most 4 passes of 256 threads); the row stays in
    // registers between the sum of squares and the scaling
    const uint16_t* e = (const uint16_t*)emb + (size_t)tok * d;
    uint4 ev[4], wv[4];
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < 4; it++) {
      const int i = (it * 256 + threadIdx.x) * 8;
      if (i >= d) continue;
      ev[it] = *(const uint4*)(e + i);
      wv[it] = *(const uint4*)(nw + i);
    }
#pragma unroll
    for (int it = 0; it < 4; it++) {
      const int i = (it * 256 + threadIdx.x) * 8;
      if (i >= d) continue;
      const uint32_t ew[4] = {ev[it].x, ev[it].y, ev[it].z, ev[it].w};
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; q++) {
        v[q] = bf2f((uint16_t)(ew[q >> 1] >> ((q & 1) * 16)));
        ss = fmaf(v[q], v[q], ss);
      }
      *(float4*)(xr + i) = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)(xr + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = sh[0] + sh[1] + sh[2] + sh[3];
    // deferred RMSNorm: the GEMM input is bf16(x * w); the consumers scale
    // by 1/rms from the row's sum of squares (here in one piece)
    if (threadIdx.x < SSQ_STRIDE) ssq[r * SSQ_STRIDE + threadIdx.x] = threadIdx.x == 0 ? ss : 0.f;
    const float inv = 1.f;
    (void)eps;
#pragma unroll
    for (int it = 0; it < 4; it++) {
      const int i = (it * 256 + threadIdx.x) * 8;
      if (i >= d) continue;
      const uint32_t ew[4] = {ev[it].x, ev[it].y, ev[it].z, ev[it].w};
      const uint32_t ww[4] = {wv[it].x, wv[it].y, wv[it].z, wv[it].w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const float v0 = bf2f((uint16_t)(ew[q] & 0xffff)) * inv * bf2f((uint16_t)(ww[q] & 0xffff));
        const float v1 = bf2f((uint16_t)(ew[q] >> 16)) * inv * bf2f((uint16_t)(ww[q] >> 16));
        o[q] = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
      }
      *(uint4*)&xnf[frag_index(r, i, MTT)] = uint4{o[0], o[1], o[2], o[3]};
    }
  } else {
    const float* e = (const float*)emb + (size_t)tok * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) xr[i] = e[i];
  }
}

void launch_assemble(int mode, const DevState* st, const int32_t* win,
                     const int32_t* pool_len, const int32_t* pool, const int32_t* prompt,
                     int M, int T, int V, int W, int N, int G, int32_t* tokens, int32_t* relpos,
                     DevState* st_w, const void* emb, int d, int bf16, float* x,
                     const uint16_t* nw, float eps, uint16_t* xnf, int MTT, float* ssq,
                     const float* rope_cos, const float* rope_sin, float* rope_rows,
                     hipStream_t s) {
  hipLaunchKernelGGL(k_assemble, dim3(M), dim3(256), 0, s, mode, st, win, pool_len, pool,
                     prompt, T, V, W, N, G, tokens, relpos, st_w, emb, d, bf16, x, nw, eps, xnf,
                     MTT, ssq, rope_cos, rope_sin, rope_rows);
}

// ---------------------------------------------------------------------------
// RMSNorm: out = x / sqrt(mean(x^2) + eps) * w, one workgroup per row

template <typename T>
__device__ inline float ldw(const void* w, int i);
template <>
__device__ inline float ldw<uint16_t>(const void* w, int i) { return bf2f(((const uint16_t*)w)[i]); }
template <>
__device__ inline float ldw<float>(const void* w, int i) { return ((const float*)w)[i]; }

__device__ inline float block_sum_256(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) sh[w] = v;
  __syncthreads();
  float t = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return t;
}

template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x, const void* w,
                                                 int d, float eps, void* out) {
  __shared__ float sh[4];
  const int r = blockIdx.x;
  const float* xr = x + (size_t)r * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss = fmaf(xr[i], xr[i], ss);
  ss = block_sum_256(ss, sh);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += 256) {
    const float v = xr[i] * inv * ldw<T>(w, i);
    if (sizeof(T) == 2) ((uint16_t*)out)[(size_t)r * d + i] = f2bf(v);
    else ((float*)out)[(size_t)r * d + i] = v;
  }
}

void launch_rmsnorm(const float* x, const void* w, int M, int d, float eps, int bf16,
                    void* out, hipStream_t s) {
  if (bf16) hipLaunchKernelGGL(k_rmsnorm<uint16_t>, dim3(M), dim3(256), 0, s, x, w, d, eps, out);
  else hipLaunchKernelGGL(k_rmsnorm<float>, dim3(M), dim3(256), 0, s, x, w, d, eps, out);
}

// ---------------------------------------------------------------------------
// n-gram pool: per lead token a list of at most G distinct (N-1)-token
// tails, oldest first.  A tail already present moves to the newest slot; a
// new tail in a full list evicts the oldest.

__device__ void pool_insert_serial(int32_t* pool_len, int32_t* pool, int N, int G, int key,
                                   const int32_t* tail) {
  if (G <= 0) return;
  const int n1 = N - 1;
  int32_t* lst = pool + (size_t)key * G * n1;
  int len = pool_len[key];
  int found = -1;
  for (int e = 0; e < len && found < 0; e++) {
    bool same = true;
    for (int i = 0; i < n1; i++) same = same && lst[e * n1 + i] == tail[i];
    if (same) found = e;
  }
  int gap;
  if (found >= 0) gap = found;
  else if (len == G) gap = 0;
  else gap = len++;
  for (int e = gap; e + 1 < len; e++)
    for (int i = 0; i < n1; i++) lst[e * n1 + i] = lst[(e + 1) * n1 + i];
  for (int i = 0; i < n1; i++) lst[(len - 1) * n1 + i] = tail[i];
  pool_len[key] = len;
}

__global__ void k_pool_insert(int32_t key, const int32_t* tail, int32_t* pool_len,
                              int32_t* pool, int N, int G) {
  if (threadIdx.x == 0) pool_insert_serial(pool_len, pool, N, G, key, tail);
}

// Every N-gram of seq[0..m) in position order: key seq[p], tail
// seq[p+1 .. p+N-1] ("Key points", "Ablation": n-grams from the prompt in
// the pool).  One lane: inserts are strictly sequential.
__global__ void k_seed_pool(const int32_t* seq, int m, int32_t* pool_len, int32_t* pool, int N,
                            int G) {
  if (threadIdx.x != 0) return;
  for (int p = 0; p + N - 1 < m; p++) pool_insert_serial(pool_len, pool, N, G, seq[p], seq + p + 1);
}

void launch_seed_pool(const int32_t* seq_dev, int m, int32_t* pool_len, int32_t* pool, int N,
                      int G, hipStream_t s) {
  hipLaunchKernelGGL(k_seed_pool, dim3(1), dim3(64), 0, s, seq_dev, m, pool_len, pool, N, G);
}

void launch_pool_insert(DevState*, int32_t key, const int32_t* tail_dev, int32_t* pool_len,
                        int32_t* pool, int N, int G, hipStream_t s) {
  hipLaunchKernelGGL(k_pool_insert, dim3(1), dim3(64), 0, s, key, tail_dev, pool_len, pool, N, G);
}

// ---------------------------------------------------------------------------
// Greedy verification + lookahead update (one 4-wave workgroup per sequence).
//   k_g = longest prefix of candidate g that follows the greedy chain:
//     cand[g][0] == argmax(row 0), cand[g][i] == argmax(row (g, i));
//   winner g* = lowest g with the largest k_g (k = 0 and g* = -1 without
//   candidates); emitted = cand[g*][0..k-1] + the next greedy token
//   (argmax of row (g*, k), or of row 0 when k = 0).
//   The new window level is the argmax of the last level's rows; column j's
//   n-gram (win[1][j], ..., win[N-1][j], new[j]) is inserted keyed by
//   win[1][j] for j = 0..W-1 in order; then the levels move down by one.

// Pool lists of the W keys a step touches are staged in LDS when they fit:
// the inserts (strictly in column order, keys may repeat) then run on LDS
// copies, and each distinct key's list is written back once.
constexpr int POOL_LDS_INTS = 6144;

// Insert tail into the LDS list lst (len entries of n1 <= 31 tokens, oldest
// first) with a group of GS lanes of one wave (GS >= G: lane e of the group
// looks after entry e); returns the new length.  Same result as
// pool_insert_serial: a tail already present is moved to the newest end,
// else it is appended, the oldest entry dropped when the list holds G.  The
// lowest matching entry wins; entries gap+1 .. len-1 then move down by one,
// each lane reading its source entry before it writes (LDS operations of one
// wave execute in program order, so every read of the move precedes every
// write of it, and the group needs no barrier).
template <int GS>
__device__ inline int pool_insert_group(int32_t* lst, int len, int n1, int G, const int32_t* tail) {
  const int lane = threadIdx.x & 63, e = lane & (GS - 1);
  const int gbase = lane & ~(GS - 1);
  bool same = e < len;
  if (same)  // entries past the length are not read
    for (int i = 0; i < n1; i++) same &= lst[e * n1 + i] == tail[i];
  const uint64_t m = (__ballot(same) >> gbase) & (GS == 64 ? ~0ull : ((1ull << GS) - 1ull));
  int gap, nlen = len;
  if (m) gap = __ffsll((unsigned long long)m) - 1;
  else if (len == G) gap = 0;
  else gap = nlen++;
  // ints [(gap + 1) n1, nlen n1) move down by n1: all reads, then all writes
  constexpr int MAXI = GS == 16 ? 16 : 31;  // G <= GS entries of n1 <= 16 (GS 16) or 31 ints
  const int from = (gap + 1) * n1, end = nlen * n1;
  int v[MAXI];
#pragma unroll
  for (int q = 0; q < MAXI; q++) {
    const int idx = from + e + q * GS;
    if (idx < end) v[q] = lst[idx];
  }
#pragma unroll
  for (int q = 0; q < MAXI; q++) {
    const int idx = from + e + q * GS;
    if (idx < end) lst[idx - n1] = v[q];
  }
  if (e < n1) lst[(nlen - 1) * n1 + e] = tail[e];
  return nlen;
}

// One workgroup of VER_T threads per sequence of the batch (its rows,
// window, pool, result).
constexpr int VER_T = 256;

__global__ __launch_bounds__(VER_T) void k_verify(DevState* st, const int32_t* __restrict__ tokens,
                                                  const int32_t* __restrict__ amax, int32_t* win,
                                                  int32_t* pool_len, int32_t* pool, int V, int W,
                                                  int N, int G, DevResult* res) {
  __shared__ int32_t ynew[256];
  __shared__ int32_t lwin[256];             // window, (N-1) x W <= 255
  __shared__ int32_t ltail[256];            // column j's tail at j * (N-1) (staged inserts)
  __shared__ int32_t tail[32];
  __shared__ int32_t lkey[256], lslot[256], llen[256], lnext[256];
  __shared__ int32_t ltok[256], lamax[256];  // the block's tokens and row argmax
  __shared__ int32_t llist[POOL_LDS_INTS];
  __shared__ int32_t best[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int n1 = N - 1;
  const int nwin = n1 * W;
  const int T = 1 + (W + G) * n1;
  const int per = G * n1;  // ints per key list
  // staged: the W lists fit in LDS and a group of at most 64 lanes covers a list
  const bool staged = G > 0 && W > 0 && W * per <= POOL_LDS_INTS && G <= 64;
  {
    const int b = blockIdx.x;
    st += b;
    tokens += (size_t)b * T;
    amax += (size_t)b * T;
    win += (size_t)b * nwin;
    pool_len += (size_t)b * V;
    pool += (size_t)b * V * per;
    res += b;
  }
  // every global read that does not depend on another goes out first
  for (int i = tid; i < T; i += VER_T) {
    ltok[i] = tokens[i];
    lamax[i] = amax[i];
  }
  for (int i = tid; i < nwin; i += VER_T) lwin[i] = win[i];
  const int nc = st->n_cand;
  __syncthreads();
  const int a0 = lamax[0];
  for (int j = tid; j < W; j += VER_T) ynew[j] = lamax[1 + (n1 - 1) * W + j];
  if (staged) {
    // lists are read whole (entries past the length are never used), so
    // the lengths and the lists load together
    for (int j = tid; j < W; j += VER_T) {
      const int key = lwin[j];
      lkey[j] = key;
      llen[j] = pool_len[key];
    }
    // every list load of the thread goes out before the first LDS store
    constexpr int MAXL = POOL_LDS_INTS / VER_T;
    int lv[MAXL];
#pragma unroll
    for (int q = 0; q < MAXL; q++) {
      const int idx = tid + q * VER_T;
      if (idx < W * per) {
        const int j = idx / per;
        lv[q] = pool[(size_t)lwin[j] * per + (idx - j * per)];
      }
    }
#pragma unroll
    for (int q = 0; q < MAXL; q++) {
      const int idx = tid + q * VER_T;
      if (idx < W * per) llist[idx] = lv[q];
    }
  }
  if (tid < 64) {
    // per-candidate accepted length, reduced to (max k, lowest g)
    int bk = -1, bg = 0x7fffffff;
    for (int g = lane; g < nc; g += 64) {
      const int base = 1 + nwin + g * n1;  // row (g, 1)
      int k = 0;
      while (k < n1) {
        const int pred = k == 0 ? a0 : lamax[base + k - 1];
        if (ltok[base + k] != pred) break;
        k++;
      }
      if (k > bk || (k == bk && g < bg)) { bk = k; bg = g; }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const int ok = __shfl_xor(bk, o), og = __shfl_xor(bg, o);
      if (ok > bk || (ok == bk && og < bg)) { bk = ok; bg = og; }
    }
    if (lane == 0) {
      best[0] = bk;
      best[1] = bg;
    }
  }
  if (staged) {
    for (int j = tid; j < W; j += VER_T) {  // first and next column with the same key
      int sl = j, nx = W;
      for (int q = 0; q < j; q++)
        if (lwin[q] == lwin[j]) { sl = q; break; }
      for (int q = W - 1; q > j; q--)
        if (lwin[q] == lwin[j]) nx = q;
      lslot[j] = sl;
      lnext[j] = nx;
    }
    for (int i = tid; i < nwin; i += VER_T) {  // tail of column j: levels 2..N-1, then the new token
      const int j = i / n1, l = i - j * n1;
      ltail[i] = l + 1 < n1 ? lwin[(l + 1) * W + j] : lamax[1 + (n1 - 1) * W + j];
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int bk = best[0], bg = best[1];
    const int k = nc > 0 ? bk : 0;
    const int gs = nc > 0 ? bg : -1;
    const int base = 1 + nwin + (gs < 0 ? 0 : gs) * n1;
    for (int i = 0; i < k; i++) res->tokens[i] = ltok[base + i];
    const int bonus = k == 0 ? a0 : lamax[base + k - 1];
    res->tokens[k] = bonus;
    for (int i = k + 1; i < 32; i++) res->tokens[i] = 0;
    res->n_emitted = k + 1;
    res->accepted = k;
    res->winner = gs;
    res->n_candidates = nc;
    const int L = st->L;
    st->L_old = L;
    st->k = k;
    st->winner = gs;
    st->L = L + k + 1;
    st->cur = bonus;
    res->kv_len = L + k + 1;
    // n-gram pool, lists not staged: insert every column's n-gram in
    // column order, one lane
    if (!staged)
      for (int j = 0; j < W; j++) {
        for (int l = 2; l <= n1; l++) tail[l - 2] = lwin[(l - 1) * W + j];
        tail[n1 - 1] = ynew[j];
        pool_insert_serial(pool_len, pool, N, G, lwin[j], tail);
      }
  }
  if (staged) {
    // staged lists: the inserts of one key in column order by one lane
    // group (key slot s by group s mod the group count), the groups side by
    // side: each walks the columns with its own cursor, so the groups of a
    // wave run their next inserts together (16-lane groups up to G = 16 and
    // N - 1 = 16 tail tokens, whole waves up to 64)
    auto inserts = [&](auto gsz) {
      constexpr int GS = decltype(gsz)::value;
      const int grp = tid / GS, ngrp = VER_T / GS;
      for (int sl = grp; sl < W; sl += ngrp) {  // uniform over the group
        if (lslot[sl] != sl) continue;  // not the first column of its key
        int len = llen[sl];
        for (int j = sl; j < W; j = lnext[j])
          len = pool_insert_group<GS>(llist + sl * per, len, n1, G, ltail + j * n1);
        if ((tid & (GS - 1)) == 0) llen[sl] = len;
      }
    };
    if (G <= 16 && n1 <= 16)
      inserts(std::integral_constant<int, 16>{});
    else
      inserts(std::integral_constant<int, 64>{});
    __syncthreads();
    for (int j = tid; j < W; j += VER_T)
      if (lslot[j] == j) pool_len[lkey[j]] = llen[j];
    for (int idx = tid; idx < W * per; idx += VER_T) {
      const int j = idx / per, rem = idx - j * per;
      if (lslot[j] == j && rem < llen[j] * n1) pool[(size_t)lkey[j] * per + rem] = llist[idx];
    }
  }
  // shift the window by one level (lwin holds the old levels)
  for (int i = tid; i < nwin; i += VER_T) {
    const int l = i / W, j = i - l * W;
    win[i] = l + 1 < n1 ? lwin[(l + 1) * W + j] : ynew[j];
  }
}

void launch_verify(DevState* st, const int32_t* tokens, const int32_t* amax, int32_t* win,
                   int32_t* pool_len, int32_t* pool, int nseq, int V, int W, int N, int G,
                   DevResult* res, hipStream_t s) {
  hipLaunchKernelGGL(k_verify, dim3(nseq), dim3(VER_T), 0, s, st, tokens, amax, win, pool_len, pool,
                     V, W, N, G, res);
}

// ---------------------------------------------------------------------------
// KV compaction: the accepted candidate rows (g*, 1..k), written at
// L_old + row by the QKV epilogue, move to L_old + 1 .. L_old + k.  Row 0 is
// already at L_old.  Sources never overlap other rows' destinations.
// Grid (layer, kv head, sequence); caches [layer][sequence][kv head][...].

template <typename E>
__global__ void k_kv_compact(const DevState* __restrict__ st, int nseq, int Hkv, int dh,
                             int max_ctx, int W, int N, E* kc, E* vtc) {
  const int layer = blockIdx.x, hk = blockIdx.y, sq = blockIdx.z;
  st += sq;
  const int k = st->k;
  if (k == 0) return;
  const int g = st->winner, L0 = st->L_old;
  const int src0 = L0 + 1 + (N - 1) * W + g * (N - 1);  // row (g, 1)
  const size_t head = ((size_t)layer * nseq + sq) * Hkv + hk;
  E* kb = kc + head * max_ctx * dh;
  E* vb = vtc + head * dh * max_ctx;
  for (int e = threadIdx.x; e < k * dh; e += blockDim.x) {
    const int i = e / dh, di = e % dh;
    kb[(size_t)(L0 + 1 + i) * dh + di] = kb[(size_t)(src0 + i) * dh + di];
    vb[(size_t)di * max_ctx + L0 + 1 + i] = vb[(size_t)di * max_ctx + src0 + i];
  }
}

void launch_kv_compact(const DevState* st, int nseq, int n_layers, int Hkv, int dh, int max_ctx,
                       int W, int N, int elem, void* k_cache, void* vt_cache, hipStream_t s) {
  dim3 grid(n_layers, Hkv, nseq);
  if (elem == 2)
    hipLaunchKernelGGL(k_kv_compact<uint16_t>, grid, dim3(256), 0, s, st, nseq, Hkv, dh, max_ctx,
                       W, N, (uint16_t*)k_cache, (uint16_t*)vt_cache);
  else
    hipLaunchKernelGGL(k_kv_compact<uint32_t>, grid, dim3(256), 0, s, st, nseq, Hkv, dh, max_ctx,
                       W, N, (uint32_t*)k_cache, (uint32_t*)vt_cache);
}

// ---------------------------------------------------------------------------
// prefill bookkeeping: commit M rows; optionally take the last row's argmax
// as the current token.

__global__ void k_advance(DevState* st, int M, const int32_t* amax, int set_cur) {
  if (threadIdx.x == 0) {
    st->L += M;
    if (set_cur) st->cur = amax[M - 1];
  }
}

void launch_advance(DevState* st, int M, const int32_t* amax, int set_cur, hipStream_t s) {
  hipLaunchKernelGGL(k_advance, dim3(1), dim3(64), 0, s, st, M, amax, set_cur);
}

}  // namespace la
