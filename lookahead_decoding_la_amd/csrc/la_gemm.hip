// Skinny-M GEMMs of the decoder forward pass: Y[M x N] = X[M x K] W^T with
// fused epilogues (logits store, residual add, RoPE + KV-cache write for the
// fused QKV projection, SwiGLU for the fused gate/up projection).
//
// The lookahead step forwards 1 + (W+G)(N-1) rows at once ("Break the
// Sequential Dependency of LLM Inference Using Lookahead Decoding", Key
// points, "Main limitation": 120 extra rows at the 7B setting), so every
// weight byte feeds ~121 multiply-adds: still below the MI355X bf16 ridge,
// so the kernel is built to stream weights at HBM rate while MFMA does the
// arithmetic on the side.
//
// bf16 kernel layout (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//   - A operand = weight tile, 16 output rows x 32 k, pre-packed so one wave
//     load is 1 KiB contiguous (16 B per lane);
//   - B operand = activation fragment, 32 k x 16 rows of X, read from L2;
//   - a workgroup (4 waves) owns 32 output rows; its waves interleave over
//     the k-steps (adjacent 1 KiB tiles stream in parallel) and are reduced
//     through LDS in a fixed order;
//   - a K split across workgroups, when the row tiles alone cannot fill 256
//     CUs, is reduced by the last-arriving workgroup in split order, so the
//     result is deterministic.
#include "la_internal.h"

namespace la {

constexpr int GEMM_NA = 2;     // 16-row A tiles per workgroup (32 rows)
constexpr int GEMM_NW = 4;     // waves per workgroup
constexpr int GEMM_THREADS = 64 * GEMM_NW;

// ---------------------------------------------------------------------------
// epilogues on a pair of adjacent output columns (n even)

template <typename ACT>
__device__ inline void store_act(void* base, size_t idx, float v);
template <>
__device__ inline void store_act<uint16_t>(void* base, size_t idx, float v) {
  ((uint16_t*)base)[idx] = f2bf(v);
}
template <>
__device__ inline void store_act<float>(void* base, size_t idx, float v) {
  ((float*)base)[idx] = v;
}

template <int EPI, typename ACT>
__device__ inline void epi_pair(const EpiArgs& ea, int t, int n, float v0, float v1) {
  if (EPI == EPI_LOGITS) {
    float* o = ea.out_f32 + (size_t)t * ea.ld_out + n;
    o[0] = v0;
    o[1] = v1;
  } else if (EPI == EPI_RESID) {
    float* o = ea.out_f32 + (size_t)t * ea.ld_out + n;
    o[0] += v0;
    o[1] += v1;
  } else if (EPI == EPI_QKV) {
    const int L = ea.st->L;
    const int dh = ea.dh;
    if (n < ea.qdim + ea.kvdim) {
      // rotate the adjacent pair (n, n+1) by angle pos * theta^(-2i/dh)
      int di = (n < ea.qdim ? n : n - ea.qdim) % dh;
      int pos = L + ea.relpos[t];
      float c = ea.rope_cos[(size_t)pos * (dh / 2) + di / 2];
      float s = ea.rope_sin[(size_t)pos * (dh / 2) + di / 2];
      float r0 = v0 * c - v1 * s, r1 = v0 * s + v1 * c;
      if (n < ea.qdim) {
        size_t o = (size_t)t * ea.qdim + n;
        store_act<ACT>(ea.out_act, o, r0);
        store_act<ACT>(ea.out_act, o + 1, r1);
      } else {
        int kv = n - ea.qdim, hk = kv / dh;
        size_t o = ((size_t)hk * ea.max_ctx + L + t) * dh + di;
        store_act<ACT>(ea.k_cache, o, r0);
        store_act<ACT>(ea.k_cache, o + 1, r1);
      }
    } else {
      int vv = n - ea.qdim - ea.kvdim, hk = vv / dh, di = vv % dh;
      size_t o = ((size_t)hk * dh + di) * ea.max_ctx + L + t;
      store_act<ACT>(ea.vt_cache, o, v0);
      store_act<ACT>(ea.vt_cache, o + ea.max_ctx, v1);
    }
  }
}

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

template <typename ACT>
__device__ inline void epi_swiglu_pair(const EpiArgs& ea, int t, int j, float g0,
                                       float g1, float u0, float u1) {
  size_t o = (size_t)t * ea.ld_out + j;
  store_act<ACT>(ea.out_act, o, silu(g0) * u0);
  store_act<ACT>(ea.out_act, o + 1, silu(g1) * u1);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel

template <int MT, int EPI>
__global__ __launch_bounds__(GEMM_THREADS) void k_gemm_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp, int K,
    int ksplit, float* __restrict__ partial, int32_t* __restrict__ counters,
    EpiArgs ea) {
  constexpr int NA = GEMM_NA, NW = GEMM_NW;
  constexpr int PER_WAVE = NA * MT * 4;  // accumulator floats per lane
  __shared__ float red[NW * PER_WAVE * 64];
  __shared__ int s_last;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wt = blockIdx.x, kz = blockIdx.y;
  const int KS = K >> 5;
  const int ks0 = (int)((long)KS * kz / ksplit);
  const int ks1 = (int)((long)KS * (kz + 1) / ksplit);
  const bf16x8* __restrict__ Wv = (const bf16x8*)Wp;
  const bf16x8* __restrict__ Xv = (const bf16x8*)X;
  const int K8 = K >> 3;
  const size_t a_base = (size_t)wt * NA * KS * 64 + l;
  const int xoff = (l & 15) * K8 + (l >> 4);

  f32x4 acc[NA][MT];
#pragma unroll
  for (int a = 0; a < NA; a++)
#pragma unroll
    for (int m = 0; m < MT; m++) acc[a][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 ac[NA], bc[MT];
  int ks = ks0 + w;
  if (ks < ks1) {
#pragma unroll
    for (int a = 0; a < NA; a++)
      ac[a] = __builtin_nontemporal_load(&Wv[a_base + ((size_t)a * KS + ks) * 64]);
#pragma unroll
    for (int m = 0; m < MT; m++) bc[m] = Xv[(size_t)m * 16 * K8 + xoff + ks * 4];
  }
  for (; ks < ks1; ks += NW) {
    const int kn = ks + NW;
    bf16x8 an[NA], bn[MT];
    if (kn < ks1) {
#pragma unroll
      for (int a = 0; a < NA; a++)
        an[a] = __builtin_nontemporal_load(&Wv[a_base + ((size_t)a * KS + kn) * 64]);
#pragma unroll
      for (int m = 0; m < MT; m++) bn[m] = Xv[(size_t)m * 16 * K8 + xoff + kn * 4];
    }
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int m = 0; m < MT; m++)
        acc[a][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ac[a], bc[m], acc[a][m], 0, 0, 0);
    if (kn < ks1) {
#pragma unroll
      for (int a = 0; a < NA; a++) ac[a] = an[a];
#pragma unroll
      for (int m = 0; m < MT; m++) bc[m] = bn[m];
    }
  }

  // intra-workgroup reduction over the 4 waves (fixed order)
#pragma unroll
  for (int a = 0; a < NA; a++)
#pragma unroll
    for (int m = 0; m < MT; m++)
#pragma unroll
      for (int v = 0; v < 4; v++)
        red[((w * NA + a) * MT + m) * 4 * 64 + v * 64 + l] = acc[a][m][v];
  __syncthreads();

  // thread (w, l) finishes token tiles m = w, w + 4, ...
  float sum[NA][(MT + NW - 1) / NW][4];
#pragma unroll
  for (int a = 0; a < NA; a++)
#pragma unroll
    for (int mi = 0; mi < (MT + NW - 1) / NW; mi++) {
      const int m = w + mi * NW;
      if (m < MT) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
          float s = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ww++)
            s += red[((ww * NA + a) * MT + m) * 4 * 64 + v * 64 + l];
          sum[a][mi][v] = s;
        }
      }
    }

  if (ksplit > 1) {
    float* my = partial + ((size_t)wt * ksplit + kz) * (NA * MT * 4 * 64);
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int mi = 0; mi < (MT + NW - 1) / NW; mi++) {
        const int m = w + mi * NW;
        if (m < MT)
#pragma unroll
          for (int v = 0; v < 4; v++) my[((a * MT + m) * 4 + v) * 64 + l] = sum[a][mi][v];
      }
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&counters[wt], 1) == ksplit - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float* base = partial + (size_t)wt * ksplit * (NA * MT * 4 * 64);
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int mi = 0; mi < (MT + NW - 1) / NW; mi++) {
        const int m = w + mi * NW;
        if (m < MT)
#pragma unroll
          for (int v = 0; v < 4; v++) {
            float s = 0.f;
            for (int z = 0; z < ksplit; z++)
              s += __builtin_nontemporal_load(&base[(size_t)z * (NA * MT * 4 * 64) +
                                                     ((a * MT + m) * 4 + v) * 64 + l]);
            sum[a][mi][v] = s;
          }
      }
    if (tid == 0) counters[wt] = 0;
  }

  // epilogue: lane l holds rows n = 16*rt + 4*(l/16) + v of token 16*m + l%16
#pragma unroll
  for (int mi = 0; mi < (MT + NW - 1) / NW; mi++) {
    const int m = w + mi * NW;
    if (m >= MT) continue;
    const int t = m * 16 + (l & 15);
    if (t >= ea.M) continue;
    if (EPI == EPI_SWIGLU) {
      // tile 0 = gate rows, tile 1 = up rows of FFN columns 16*wt ..
      const int j = wt * 16 + (l >> 4) * 4;
      epi_swiglu_pair<uint16_t>(ea, t, j, sum[0][mi][0], sum[0][mi][1], sum[1][mi][0], sum[1][mi][1]);
      epi_swiglu_pair<uint16_t>(ea, t, j + 2, sum[0][mi][2], sum[0][mi][3], sum[1][mi][2], sum[1][mi][3]);
    } else {
#pragma unroll
      for (int a = 0; a < NA; a++) {
        const int n = (wt * NA + a) * 16 + (l >> 4) * 4;
        epi_pair<EPI, uint16_t>(ea, t, n, sum[a][mi][0], sum[a][mi][1]);
        epi_pair<EPI, uint16_t>(ea, t, n + 2, sum[a][mi][2], sum[a][mi][3]);
      }
    }
  }
}

int gemm_bf16_tiles(int N) { return N / (16 * GEMM_NA); }

int gemm_bf16_ksplit(int N, int K) {
  int tiles = gemm_bf16_tiles(N), KS = K / 32, ks = 1;
  while (tiles * ks < 512 && KS / (ks * 2) >= 16) ks *= 2;
  return ks;
}

size_t gemm_bf16_partial_floats(int N, int M, int ksplit) {
  int MT = (M + 15) / 16;
  return ksplit > 1 ? (size_t)gemm_bf16_tiles(N) * ksplit * GEMM_NA * MT * 4 * 64 : 0;
}

template <int EPI>
static void launch_mt(int MT, dim3 grid, const uint16_t* X, const uint16_t* Wp,
                      int K, int ksplit, float* partial, int32_t* counters,
                      const EpiArgs& ea, hipStream_t s) {
#define LA_GEMM_CASE(mt)                                                         \
  case mt:                                                                       \
    hipLaunchKernelGGL((k_gemm_bf16<mt, EPI>), grid, dim3(GEMM_THREADS), 0, s, X, \
                       Wp, K, ksplit, partial, counters, ea);                    \
    break;
  switch (MT) {
    LA_GEMM_CASE(1) LA_GEMM_CASE(2) LA_GEMM_CASE(3) LA_GEMM_CASE(4)
    LA_GEMM_CASE(5) LA_GEMM_CASE(6) LA_GEMM_CASE(7) LA_GEMM_CASE(8)
    LA_GEMM_CASE(9) LA_GEMM_CASE(10) LA_GEMM_CASE(11) LA_GEMM_CASE(12)
    LA_GEMM_CASE(13) LA_GEMM_CASE(14) LA_GEMM_CASE(15) LA_GEMM_CASE(16)
    default: break;
  }
#undef LA_GEMM_CASE
}

void launch_gemm_bf16(int epi, const uint16_t* X, const uint16_t* Wp, int K, int N,
                      int M, int ksplit, float* partial, int32_t* counters,
                      const EpiArgs& ea, hipStream_t s) {
  const int MT = (M + 15) / 16;
  dim3 grid(gemm_bf16_tiles(N), ksplit);
  switch (epi) {
    case EPI_LOGITS: launch_mt<EPI_LOGITS>(MT, grid, X, Wp, K, ksplit, partial, counters, ea, s); break;
    case EPI_RESID: launch_mt<EPI_RESID>(MT, grid, X, Wp, K, ksplit, partial, counters, ea, s); break;
    case EPI_QKV: launch_mt<EPI_QKV>(MT, grid, X, Wp, K, ksplit, partial, counters, ea, s); break;
    case EPI_SWIGLU: launch_mt<EPI_SWIGLU>(MT, grid, X, Wp, K, ksplit, partial, counters, ea, s); break;
  }
}

// ---------------------------------------------------------------------------
// repack row-major bf16 weights into A-operand tiles

__global__ void k_repack_bf16(const uint16_t* __restrict__ src, int rows, int K,
                              uint16_t* __restrict__ dst, int rt_offset, int rt_mult) {
  const int KS = K >> 5;
  const size_t lanes = (size_t)(rows / 16) * KS * 64;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < lanes;
       i += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const size_t tile = i >> 6;
    const int ks = (int)(tile % KS);
    const int rt = (int)(tile / KS);
    const int row = rt * 16 + (l & 15), col = ks * 32 + (l >> 4) * 8;
    const uint4 v = *(const uint4*)(src + (size_t)row * K + col);
    const size_t prt = (size_t)rt_offset + (size_t)rt * rt_mult;
    *(uint4*)(dst + ((prt * KS + ks) * 64 + l) * 8) = v;
  }
}

void launch_repack_bf16(const uint16_t* src, int rows, int K, uint16_t* dst,
                        int rt_offset, int rt_mult, hipStream_t s) {
  size_t lanes = (size_t)(rows / 16) * (K / 32) * 64;
  int blocks = (int)((lanes + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_repack_bf16, dim3(blocks), dim3(256), 0, s, src, rows, K, dst,
                     rt_offset, rt_mult);
}

// ---------------------------------------------------------------------------
// fp32 kernel (small models): one thread per (row, output pair)

template <int EPI>
__global__ void k_gemm_f32(const float* __restrict__ X, const float* __restrict__ W,
                           const float* __restrict__ W2, int K, int N, int M, EpiArgs ea) {
  const int t = blockIdx.y;
  const int n = 2 * (blockIdx.x * blockDim.x + threadIdx.x);
  if (n >= N || t >= M) return;
  const float* x = X + (size_t)t * K;
  const float* w0 = W + (size_t)n * K;
  const float* w1 = w0 + K;
  float s0 = 0.f, s1 = 0.f;
  for (int k = 0; k < K; k++) {
    s0 = fmaf(x[k], w0[k], s0);
    s1 = fmaf(x[k], w1[k], s1);
  }
  if (EPI == EPI_SWIGLU) {
    const float* u0p = W2 + (size_t)n * K;
    const float* u1p = u0p + K;
    float u0 = 0.f, u1 = 0.f;
    for (int k = 0; k < K; k++) {
      u0 = fmaf(x[k], u0p[k], u0);
      u1 = fmaf(x[k], u1p[k], u1);
    }
    epi_swiglu_pair<float>(ea, t, n, s0, s1, u0, u1);
  } else {
    epi_pair<EPI, float>(ea, t, n, s0, s1);
  }
}

void launch_gemm_f32(int epi, const float* X, const float* W, const float* W2, int K,
                     int N, int M, const EpiArgs& ea, hipStream_t s) {
  dim3 grid((N / 2 + 63) / 64, M), block(64);
  switch (epi) {
    case EPI_LOGITS: hipLaunchKernelGGL(k_gemm_f32<EPI_LOGITS>, grid, block, 0, s, X, W, W2, K, N, M, ea); break;
    case EPI_RESID: hipLaunchKernelGGL(k_gemm_f32<EPI_RESID>, grid, block, 0, s, X, W, W2, K, N, M, ea); break;
    case EPI_QKV: hipLaunchKernelGGL(k_gemm_f32<EPI_QKV>, grid, block, 0, s, X, W, W2, K, N, M, ea); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_f32<EPI_SWIGLU>, grid, block, 0, s, X, W, W2, K, N, M, ea); break;
  }
}

}  // namespace la
