// Skinny-M GEMMs of the decoder forward pass, Y[M x N] = X[M x K] W^T.
//
// The lookahead step forwards 1 + (W+G)(N-1) rows at once ("Break the
// Sequential Dependency of LLM Inference Using Lookahead Decoding", Key
// points, "Main limitation": 120 extra rows at the 7B setting), so each
// weight byte feeds ~121 multiply-adds: still under the MI355X bf16 ridge,
// so the kernel is built to stream weights while MFMA works on the side.
//
// bf16 kernels (gfx950, wave64, v_mfma_f32_16x16x32_bf16), chosen by the
// pass's rows:
//   - A operand = weights, pre-packed in 16-row x 32-k tiles so one wave
//     load is 1 KiB contiguous; B operand = activations, stored by their
//     producers in the fragment layout (la_epilogue.h) so one fragment is
//     1 KiB contiguous;
//   - k_gemm_dma (4 or more token tiles): a workgroup of 8 (12) waves owns
//     128 (192) output rows, one 16-row tile per wave; all waves walk the
//     same k-steps, so each activation fragment is fetched once per
//     workgroup; weights and fragments go straight into an LDS ring
//     (global_load_lds), several stages deep;
//   - k_gemm_bf16 (2-3 token tiles): the same workgroup shape with a ring of
//     weight stages in VGPRs and the fragments shared through LDS;
//   - when the row tiles alone cannot fill 256 CUs, K is split across
//     workgroups; each split writes fp32 partial sums and a reduce kernel
//     (which also applies the epilogue) adds them in split order, so
//     results are deterministic and no workgroup waits on another;
//   - k_gemv_bf16 (at most 12 rows, one token tile): one workgroup per
//     16-row weight tile over all of K, its waves summed through LDS, the
//     epilogue fused: no partial sums and no reduce kernel.
#include <algorithm>

#include "la_epilogue.h"

namespace la {

constexpr int G_NW = 8;                 // waves per workgroup
constexpr int G_ROWS = G_NW * 16;       // output rows per workgroup
constexpr int G_D = 3;                  // weight stages in the ring

// Writes fp32 partial sums P[kz][t][n] of K split kz.
template <int MT, int J>
__global__ __launch_bounds__(G_NW * 64) void k_gemm_bf16(
    const uint16_t* __restrict__ X, int MTT, const uint16_t* __restrict__ Wp, int K,
    int ksplit, float* __restrict__ P, int N, int M) {
  constexpr int NF = J * MT;                       // B fragments per stage
  constexpr int FPW = (NF + G_NW - 1) / G_NW;      // of them loaded per wave
  constexpr int D = G_D;
  __shared__ bf16x8 xs[2][NF][64];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wt = blockIdx.x, kz = blockIdx.y;
  const int KS = K >> 5;
  const int ks0 = KS * kz / ksplit;  // KS * ksplit stays far below 2^31
  const int nst = (KS * (kz + 1) / ksplit - ks0) / J;
  const bf16x8* __restrict__ Xv = (const bf16x8*)X;
  const bf16x8* __restrict__ wp =
      (const bf16x8*)Wp + ((size_t)(wt * G_NW + w) * KS) * 64 + l;

  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 ra[D][J], rx[D][FPW];

  // stage st: J k-steps; this wave's weight tiles and its share of the
  // J*MT activation fragments
#define LA_ISSUE(slot, st)                                                        \
  {                                                                               \
    const int kb_ = ks0 + (st) * J;                                               \
    _Pragma("unroll") for (int j = 0; j < J; j++)                                 \
        ra[slot][j] = __builtin_nontemporal_load(&wp[(size_t)(kb_ + j) * 64]);    \
    _Pragma("unroll") for (int q = 0; q < FPW; q++) {                             \
      const int f = w + q * G_NW;                                                 \
      if (NF % G_NW == 0 || f < NF)                                               \
        rx[slot][q] = Xv[((size_t)(kb_ + f / MT) * MTT + (f % MT)) * 64 + l];     \
    }                                                                             \
  }
#define LA_PUTX(slot, buf)                                                        \
  {                                                                               \
    _Pragma("unroll") for (int q = 0; q < FPW; q++) {                             \
      const int f = w + q * G_NW;                                                 \
      if (NF % G_NW == 0 || f < NF) xs[buf][f][l] = rx[slot][q];                  \
    }                                                                             \
  }
#define LA_MMAS(slot, buf)                                                        \
  {                                                                               \
    _Pragma("unroll") for (int j = 0; j < J; j++) {                               \
      bf16x8 b_[MT];                                                              \
      _Pragma("unroll") for (int m = 0; m < MT; m++) b_[m] = xs[buf][j * MT + m][l]; \
      _Pragma("unroll") for (int m = 0; m < MT; m++)                              \
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[slot][j], b_[m], acc[m], 0, 0, 0); \
    }                                                                             \
  }

#pragma unroll
  for (int s = 0; s < D; s++)
    if (s < nst) LA_ISSUE(s, s);
  if (nst > 0) LA_PUTX(0, 0);
  __syncthreads();
  int st = 0;
  // steady state: every stage issues the stage D ahead; no branches, so
  // loads of later stages stay in flight across the MFMAs
  for (; st + 2 * D <= nst; st += D) {
#pragma unroll
    for (int s = 0; s < D; s++) {
      LA_PUTX((s + 1) % D, (st + s + 1) & 1);
      LA_MMAS(s, (st + s) & 1);
      LA_ISSUE(s, st + s + D);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
  }
  for (; st < nst; st += D) {
#pragma unroll
    for (int s = 0; s < D; s++) {
      if (st + s < nst) {
        if (st + s + 1 < nst) LA_PUTX((s + 1) % D, (st + s + 1) & 1);
        LA_MMAS(s, (st + s) & 1);
        if (st + s + D < nst) LA_ISSUE(s, st + s + D);
      }
      __syncthreads();
    }
  }
#undef LA_ISSUE
#undef LA_PUTX
#undef LA_MMAS

  // lane holds rows n = 16*tile + 4*(l/16) + v of token 16*m + l%16
  float* out = P + (size_t)kz * M * N;
  const int n = (wt * G_NW + w) * 16 + (l >> 4) * 4;
#pragma unroll
  for (int m = 0; m < MT; m++) {
    const int t = m * 16 + (l & 15);
    if (t < M) *(f32x4*)&out[(size_t)t * N + n] = acc[m];
  }
}

// The same product with every operand loaded straight into LDS
// (global_load_lds, 1 KiB per wave instruction): no staging registers, so
// the ring can hold D stages (each J k-steps of this workgroup's NW weight
// tiles and the J*MT activation fragments) and every wave only waits for
// the stage it is about to use.  One barrier per stage: after it, every
// wave has finished the previous stage, whose slot is refilled.
// OUT == 0: workgroup wt owns weight tiles NW*wt .. NW*wt + NW-1.
// OUT == 1 (fused gate/up + SwiGLU; gate tile i and up tile i are tiles 2i
// and 2i + 1): the N/32 tile pairs are dealt to the grid's workgroups as
// evenly as possible, up to NW/2 pairs each, so that every CU streams
// about the same weight bytes (with 8-wave groups at 688 pairs, 172
// workgroups left 84 CUs idle); a wave without a pair loads its group's
// last pair again (an L2 hit beside the wave that owns it) and stores
// nothing.
template <int MT, int J, int OUT, bool XP, int NW = G_NW>
__global__ __launch_bounds__(NW * 64) void k_gemm_dma(
    const uint16_t* __restrict__ X, int MTT, const uint16_t* __restrict__ Wp, int K,
    int ksplit, float* __restrict__ P, int N, int M, uint16_t* __restrict__ A,
    const float* __restrict__ ssq, int ssn, float eps) {
  constexpr int NF = J * MT;                   // activation fragments per stage
  constexpr int FPW = (NF + NW - 1) / NW;  // of them loaded per wave
  constexpr int LPS = J + FPW;             // load instructions per thread per stage
  constexpr int WKB = NW * J;              // weight KiB per stage
  constexpr int STAGE = (WKB + NF) * 1024;
  constexpr int D = STAGE * 4 <= 160 * 1024 ? 4 : 3;
  static_assert(D * STAGE <= 160 * 1024 && (D - 2) * LPS < 64, "ring");
  static_assert(OUT == 0 || (NW % 2 == 0 && D * STAGE >= (NW / 2) * MT * 64 * 16), "LDS exchange");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[D * STAGE];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wt = blockIdx.x, kz = blockIdx.y;
  const int KS = K >> 5;
  const int ks0 = KS * kz / ksplit;  // KS * ksplit stays far below 2^31
  const int nst = (KS * (kz + 1) / ksplit - ks0) / J;
  // pairs [p0, p1) of a fused gate/up workgroup; wave w's weight tile
  int p0 = 0, p1 = 0, tile = wt * NW + w;
  if constexpr (OUT == 1) {
    const int pairs = N >> 5, base = pairs / (int)gridDim.x, extra = pairs % (int)gridDim.x;
    p0 = wt * base + min(wt, extra);
    p1 = p0 + base + (wt < extra ? 1 : 0);
    tile = 2 * min(p0 + (w >> 1), p1 - 1) + (w & 1);
  }
  const uint16_t* wb = Wp + (size_t)tile * KS * 512 + l * 8;

  // stage st into ring slot b; past the end the last stage is re-issued
  // (same count of loads every stage), never read.  Weights are read once:
  // nontemporal (aux bit 1, "nt"), which measured a few percent faster; the
  // activation fragments, re-read by every workgroup, keep the default
  // policy so they stay in L2.
  // The fused gate/up GEMM and, up to 8 token tiles, the 8-split GEMMs (no
  // fragment prefetch) walk each workgroup's K range from a different
  // starting stage (rotated by its share of the range, wrapping around), so
  // that the workgroups of a launch do not all read the same offset of their
  // weight tiles at the same moment.  Measured (same-box A/Bs, 7B shapes, us
  // per launch): 121 rows, gate/up 49.2 -> 48.8, down 23.4 -> 22.9; 201
  // rows, gate/up 84.5 -> 81.2 but down 35.3 -> 44.5 (161 rows: 30.7 ->
  // 37.2), so the 8-split GEMMs rotate only up to 8 token tiles; QKV (2
  // splits, prefetched fragments) 27.3 -> 27.6 at 121 rows keeps the plain
  // order.  The order is fixed per workgroup, so the sums do not depend on
  // timing.
  constexpr bool ROT = OUT == 1 || (!XP && MT <= 8);
  const int rot = ROT ? (int)(((uint32_t)wt * (uint32_t)nst) / gridDim.x) : 0;
  auto issue = [&](int st, int b) {
    st = min(st, nst - 1) + rot;
    if (st >= nst) st -= nst;
    const int kb = ks0 + st * J;
    unsigned char* sb = lds + b * STAGE;
#pragma unroll
    for (int j = 0; j < J; j++)
      __builtin_amdgcn_global_load_lds((const void*)(wb + (size_t)(kb + j) * 512),
                                       (__attribute__((address_space(3))) void*)(sb + (w * J + j) * 1024),
                                       16, 0, 2);
#pragma unroll
    for (int q = 0; q < FPW; q++) {
      const int f = (w + q * NW) % NF;  // waves past NF repeat a fragment: same bytes, same slot
      __builtin_amdgcn_global_load_lds(
          (const void*)(X + ((size_t)(kb + f / MT) * MTT + f % MT) * 512 + l * 8),
          (__attribute__((address_space(3))) void*)(sb + (WKB + f) * 1024), 16, 0, 0);
    }
  };

  // The activation fragments were written by the previous kernel, so no
  // XCD's L2 holds them, and every stage would wait on L2 misses that all
  // of the XCD's workgroups share (measured: the fused gate/up GEMM takes
  // 48 us after itself, 52-53 us after a kernel that rewrote its input,
  // unchanged after one that wrote other memory).  With XP (at least 4
  // token tiles and at most 2 K splits: large fragment ranges per
  // workgroup; no gain measured with 8 splits) each workgroup touches one
  // slice of its K range's fragments right after issuing the ring's first
  // stage, 8 lanes per 128-byte line so that a load instruction covers 8
  // lines like any coalesced load: workgroups are dealt to the 8 XCDs
  // round robin, so the workgroups of one K range on one XCD (grid x index
  // / 8 = slice) touch the whole range once between them and their L2
  // holds it before the ring needs it.  Every thread issues exactly XPF
  // such loads (lines past its slice repeat the slice's last line), so the
  // first stage's wait can count them; the values are consumed only after
  // the main loop.
  constexpr int XPF = XP ? 8 : 0;  // prefetch loads per thread (64 KiB per workgroup)
  static_assert((D - 2) * LPS + XPF < 64 && (D - 1) * LPS + XPF < 64, "vmcnt");
  uint32_t xpf[XP ? XPF : 1];
  auto prefetch = [&]() {
    if constexpr (XP) {
      const uint32_t nsl = max(gridDim.x >> 3, 1u), sl = min((uint32_t)wt >> 3, nsl - 1);
      // the K range's k-steps hold MTT tiles of 8 lines each; the first MT
      // tiles of every k-step are read
      const char* xr = (const char*)(X + (size_t)ks0 * MTT * 512);
      const uint32_t lines = (uint32_t)(nst * J) * MT * 8;
      const uint32_t b0 = lines * sl / nsl, b1 = lines * (sl + 1) / nsl;
#pragma unroll
      for (int i = 0; i < XPF; i++) {
        const uint32_t ln = min(b0 + (uint32_t)((i * NW + w) * 8 + (l >> 3)), max(b1, 1u) - 1);
        const uint32_t kk = ln / (MT * 8), r = ln - kk * (MT * 8);
        xpf[i] = *(const uint32_t*)(xr + ((size_t)kk * MTT * 8 + r) * 128 + (l & 7) * 16);
      }
    }
  };

  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue(0, 0);
  prefetch();
#pragma unroll
  for (int i = 1; i < D - 1; i++) issue(i, i);
  for (int st = 0; st < nst; st++) {
    // this thread's part of stage st has landed (stage 0: the XPF
    // prefetch loads issued after it may still be in flight)
    if (st == 0)
      wait_vm<(D - 2) * LPS + XPF>();
    else
      wait_vm<(D - 2) * LPS>();
    lds_barrier();  // ... everyone's; and stage st-1 is consumed
    issue(st + D - 1, (st + D - 1) % D);
    const unsigned char* sb = lds + (st % D) * STAGE;
#pragma unroll
    for (int j = 0; j < J; j++) {
      const bf16x8 a = *(const bf16x8*)(sb + (w * J + j) * 1024 + l * 16);
      bf16x8 b[MT];
#pragma unroll
      for (int m = 0; m < MT; m++) b[m] = *(const bf16x8*)(sb + (WKB + j * MT + m) * 1024 + l * 16);
#pragma unroll
      for (int m = 0; m < MT; m++) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[m], acc[m], 0, 0, 0);
    }
  }
  wait_vm<0>();  // drain the re-issued stages before the LDS is reused or freed
  if constexpr (XP) {
#pragma unroll
    for (int i = 0; i < XPF; i++) asm volatile("" ::"v"(xpf[i]));  // keep the prefetch loads
  }

  // lane holds rows n = 16*tile + 4*(l/16) + v of token 16*m + l%16
  if (OUT == 0) {
    float* out = P + (size_t)kz * M * N;
    const int n = tile * 16 + (l >> 4) * 4;
#pragma unroll
    for (int m = 0; m < MT; m++) {
      const int t = m * 16 + (l & 15);
      if (t < M) *(f32x4*)&out[(size_t)t * N + n] = acc[m];
    }
  } else {
    // wave 2i holds gate rows, wave 2i+1 the matching up rows (FFN tile
    // p0 + i); the up values pass through the (idle) ring.  The input
    // rows were not normalized: both products take the row's 1/rms here.
    f32x4* ex = (f32x4*)lds;
    float* invs = (float*)(lds + (NW / 2) * MT * 64 * 16);  // 1/rms of each token row
    static_assert(OUT == 0 || D * STAGE >= (NW / 2) * MT * 64 * 16 + MT * 16 * 4, "LDS");
    lds_barrier();
    for (int t = tid; t < M; t += NW * 64) invs[t] = row_inv_rms(ssq, ssn, t, K, eps);
    if (w & 1) {
#pragma unroll
      for (int m = 0; m < MT; m++) ex[((w >> 1) * MT + m) * 64 + l] = acc[m];
    }
    __syncthreads();
    if (!(w & 1) && p0 + (w >> 1) < p1) {
      const int j = (p0 + (w >> 1)) * 16 + (l >> 4) * 4;
#pragma unroll
      for (int m = 0; m < MT; m++) {
        const int t = m * 16 + (l & 15);
        if (t >= M) continue;
        const float inv = invs[t];
        const f32x4 u = ex[((w >> 1) * MT + m) * 64 + l] * inv;
        const f32x4 gt = acc[m] * inv;
        const size_t o = frag_index(t, j, MTT);
        uint2 pk;
        pk.x = (uint32_t)f2bf(silu(gt[0]) * u[0]) | ((uint32_t)f2bf(silu(gt[1]) * u[1]) << 16);
        pk.y = (uint32_t)f2bf(silu(gt[2]) * u[2]) | ((uint32_t)f2bf(silu(gt[3]) * u[3]) << 16);
        *(uint2*)&A[o] = pk;
      }
    }
  }
}

// K split of a plain GEMM for a step of `rows` rows, with at least 6
// k-steps per split.
//  - From 4 token tiles on (the LDS-direct kernel, every workgroup loading
//    its K range's activation fragments): the largest split count that
//    keeps the workgroups within one round on the 256 CUs (tiles * ks <=
//    256); more would start a second round on part of the CUs for no
//    smaller share of K per CU, plus partial-sum traffic (13B O and down:
//    4 splits instead of 8, 34B QKV 2 instead of 4: steps 0.8% faster).
//  - Below (one-token decode: a workgroup's work is nearly all weights):
//    the smallest split count that reaches 192 workgroups; there more
//    workgroups are only more parallelism (the one-round rule made 13B and
//    34B plain decode 4-6% slower).
GemmPlan gemm_bf16_plan(int N, int K, int rows) {
  GemmPlan p;
  const int tiles = N / G_ROWS, KS = K / 32;
  const bool one_round = (rows + 15) / 16 >= 4;
  p.ksplit = 1;
  p.J = KS % 2 == 0 ? 2 : 1;
  const int cands[] = {2, 4, 8, 16};
  for (int ks : cands) {
    if (KS % ks) continue;
    const int per = KS / ks;
    if (per < 6) break;
    if (one_round && tiles * ks > 256) break;
    if (!one_round && tiles * p.ksplit >= 192) break;
    p.ksplit = ks;
    p.J = per % 2 == 0 ? 2 : 1;
  }
  return p;
}

template <int J>
static void launch_j(int MT, dim3 grid, const uint16_t* X, int MTT, const uint16_t* Wp, int K,
                     int ks, float* P, int N, int M, hipStream_t s) {
#define LA_GEMM_CASE(mt)                                                                     \
  case mt:                                                                                   \
    hipLaunchKernelGGL((k_gemm_bf16<mt, J>), grid, dim3(G_NW * 64), 0, s, X, MTT, Wp, K, ks, \
                       P, N, M);                                                             \
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

template <int J>
static void launch_dma_part(int MT, dim3 grid, const uint16_t* X, int MTT, const uint16_t* Wp,
                            int K, int ks, float* P, int N, int M, hipStream_t s) {
#define LA_GEMM_CASE(mt)                                                                         \
  case mt:                                                                                       \
    if (ks <= 2)                                                                                 \
      hipLaunchKernelGGL((k_gemm_dma<mt, J, 0, true>), grid, dim3(G_NW * 64), 0, s, X, MTT, Wp, \
                         K, ks, P, N, M, nullptr, nullptr, 0, 0.f);                              \
    else                                                                                         \
      hipLaunchKernelGGL((k_gemm_dma<mt, J, 0, false>), grid, dim3(G_NW * 64), 0, s, X, MTT, Wp, \
                         K, ks, P, N, M, nullptr, nullptr, 0, 0.f);                              \
    break;
  switch (MT) {
    LA_GEMM_CASE(4) LA_GEMM_CASE(5) LA_GEMM_CASE(6) LA_GEMM_CASE(7)
    LA_GEMM_CASE(8) LA_GEMM_CASE(9) LA_GEMM_CASE(10) LA_GEMM_CASE(11)
    LA_GEMM_CASE(12) LA_GEMM_CASE(13) LA_GEMM_CASE(14) LA_GEMM_CASE(15)
    LA_GEMM_CASE(16)
    default: break;
  }
#undef LA_GEMM_CASE
}

void launch_gemm_bf16(const uint16_t* X, int MTT, const uint16_t* Wp, int K, int N, int M,
                      const GemmPlan& plan, float* P, hipStream_t s) {
  const int MT = (M + 15) / 16;
  dim3 grid(N / G_ROWS, plan.ksplit);
  // from 4 token tiles on, the LDS-direct kernel (deeper ring) is faster;
  // below, the register-ring kernel
  if (MT >= 4) {
    if (plan.J == 2) launch_dma_part<2>(MT, grid, X, MTT, Wp, K, plan.ksplit, P, N, M, s);
    else launch_dma_part<1>(MT, grid, X, MTT, Wp, K, plan.ksplit, P, N, M, s);
    return;
  }
  if (plan.J == 2) launch_j<2>(MT, grid, X, MTT, Wp, K, plan.ksplit, P, N, M, s);
  else launch_j<1>(MT, grid, X, MTT, Wp, K, plan.ksplit, P, N, M, s);
}

template <int J, int NW>
static void launch_dma_swiglu(int MT, dim3 grid, const uint16_t* X, int MTT, const uint16_t* Wp,
                              int K, int N, int M, uint16_t* A, const float* ssq, int ssn,
                              float eps, hipStream_t s) {
#define LA_GEMM_CASE(mt)                                                                        \
  case mt:                                                                                      \
    hipLaunchKernelGGL((k_gemm_dma<mt, J, 1, (mt >= 4), NW>), grid, dim3(NW * 64), 0, s, X, MTT, \
                       Wp, K, 1, nullptr, N, M, A, ssq, ssn, eps);                              \
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

// Fused gate/up: 8-wave workgroups, 4 gate/up tile pairs each, while that
// takes at most 256 workgroups (one round on the CUs).  Beyond that (more
// than 1024 pairs: 34B shape, 1376) the pairs are dealt evenly over 256
// 12-wave workgroups, up to 6 pairs each, instead of a second round on
// part of the CUs (34B: gate/up 148 -> 120 us, step 15.8 -> 14.4 ms).
// Spreading fewer pairs over more workgroups measured no gain: every
// workgroup loads all activation fragments (13B, 864 pairs over 256
// workgroups instead of 216: 58 -> 66 us; 7B, 688 pairs with 6-wave
// groups: within +-1 us).
void launch_gemm_bf16_swiglu(const uint16_t* X, int MTT, const uint16_t* Wp, int K, int N, int M,
                             int J, uint16_t* A, const float* ssq, int ssn, float eps,
                             hipStream_t s) {
  const int MT = (M + 15) / 16;
  const int pairs = N / 32;
  if (pairs > 1024 && pairs <= 6 * 256) {
    launch_dma_swiglu<1, 12>(MT, dim3(256, 1), X, MTT, Wp, K, N, M, A, ssq, ssn, eps, s);
    return;
  }
  const dim3 grid(pairs / 4, 1);  // N % 128 == 0
  if (J == 2) launch_dma_swiglu<2, 8>(MT, grid, X, MTT, Wp, K, N, M, A, ssq, ssn, eps, s);
  else launch_dma_swiglu<1, 8>(MT, grid, X, MTT, Wp, K, N, M, A, ssq, ssn, eps, s);
}

// ---------------------------------------------------------------------------
// reduce kernels: sum the K-split partials P[z][t][n] in split order and
// apply the epilogue.  One workgroup per token row.

// Each thread owns 8 adjacent output columns: two float4 loads per split,
// and for fragment-layout outputs one 16-byte store (8 adjacent k).

__device__ inline void load8(const float* p, float* v) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ inline uint4 pack8(const float* v) {
  uint4 r;
  r.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  r.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  r.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
  r.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
  return r;
}

// Fused QKV: sum the K splits of one 128-column block (one q, k or v head)
// for 32 tokens, then RoPE + store q (row-major) or k (cache rows), or
// transpose v through LDS so that the V^T cache rows (positions of one
// dimension) are written as contiguous runs.  Thread: token tid/8, columns
// 16*(tid%8) .. +16 of the block.  Every load the thread needs (the KS
// partials, the row's sums of squares, the rotary factors, the committed
// length) is issued before the first is used: one memory round trip.
constexpr int RQ_TOK = 32;

template <int KS>
__global__ __launch_bounds__(256) void k_red_qkv(const float* __restrict__ P, int ks, int N,
                                                 int M, EpiArgs ea) {
  __shared__ float vt[RQ_TOK][128 + 1];
  const int cb = blockIdx.x, tid = threadIdx.x;
  const int tl = tid >> 3, c0 = (tid & 7) * 16;
  const int t = blockIdx.y * RQ_TOK + tl;
  const int n0 = cb * 128 + c0;
  const bool is_v = cb * 128 >= ea.qdim + ea.kvdim;
  const int tc = min(t, M - 1);  // rows past M repeat a valid row, never stored
  // block row tq of sequence b (its state and caches)
  const int b = tc / ea.rps, tq = tc - b * ea.rps;
  const int L = ea.st[b].L;
  constexpr int NZ = KS > 0 ? KS : 1;
  float4 pz[NZ][4];
#pragma unroll
  for (int z = 0; z < NZ; z++)
#pragma unroll
    for (int e = 0; e < 4; e++) pz[z][e] = *(const float4*)(P + ((size_t)z * M + tc) * N + n0 + 4 * e);
  static_assert(SSQ_STRIDE == 8, "sums of squares: two float4 per row");
  const float4 q0 = *(const float4*)(ea.ssq + tc * SSQ_STRIDE);
  const float4 q1 = *(const float4*)(ea.ssq + tc * SSQ_STRIDE + 4);
  float4 rc0, rc1, rs0, rs1;  // rotary factors of pairs c0/2 .. c0/2 + 7
  if (!is_v) {
    const float* cs = ea.rope_rows + (size_t)tc * 128 + c0 / 2;
    rc0 = *(const float4*)cs;
    rc1 = *(const float4*)(cs + 4);
    rs0 = *(const float4*)(cs + 64);
    rs1 = *(const float4*)(cs + 68);
  }
  float v[16];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    v[4 * e] = pz[0][e].x; v[4 * e + 1] = pz[0][e].y;
    v[4 * e + 2] = pz[0][e].z; v[4 * e + 3] = pz[0][e].w;
  }
#pragma unroll
  for (int z = 1; z < NZ; z++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      v[4 * e] += pz[z][e].x; v[4 * e + 1] += pz[z][e].y;
      v[4 * e + 2] += pz[z][e].z; v[4 * e + 3] += pz[z][e].w;
    }
  if constexpr (KS == 0) {  // any other split count: the remaining splits in order
    for (int z = 1; z < ks; z++) {
      const float* pr = P + ((size_t)z * M + tc) * N + n0;
#pragma unroll
      for (int e = 0; e < 16; e += 4) {
        const float4 a = *(const float4*)(pr + e);
        v[e] += a.x; v[e + 1] += a.y; v[e + 2] += a.z; v[e + 3] += a.w;
      }
    }
  }
  {
    // the input rows were not normalized (deferred RMSNorm); chunk sums in
    // order, as row_inv_rms adds them
    const float qs[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (i < ea.ssn) sq += qs[i];
    const float inv = 1.f / sqrtf(sq / (float)ea.dmodel + ea.eps);
#pragma unroll
    for (int e = 0; e < 16; e++) v[e] *= inv;
  }
  if (!is_v) {
    // rotary angle of pair i (dims 2i, 2i+1 of the head) at pos
    const float cs[8] = {rc0.x, rc0.y, rc0.z, rc0.w, rc1.x, rc1.y, rc1.z, rc1.w};
    const float sn[8] = {rs0.x, rs0.y, rs0.z, rs0.w, rs1.x, rs1.y, rs1.z, rs1.w};
    uint16_t o[16];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float c = cs[e], s = sn[e];
      o[2 * e] = f2bf(v[2 * e] * c - v[2 * e + 1] * s);
      o[2 * e + 1] = f2bf(v[2 * e] * s + v[2 * e + 1] * c);
    }
    if (t < M) {
      uint16_t* dst;
      if (n0 < ea.qdim) {
        dst = (uint16_t*)ea.out_act + (size_t)t * ea.qdim + n0;
      } else {
        const int hk = (n0 - ea.qdim) >> 7;
        dst = (uint16_t*)ea.k_cache + b * ea.kv_seq + ((size_t)hk * ea.max_ctx + L + tq) * 128 + c0;
      }
      uint4 a, b;
      a.x = o[0] | ((uint32_t)o[1] << 16); a.y = o[2] | ((uint32_t)o[3] << 16);
      a.z = o[4] | ((uint32_t)o[5] << 16); a.w = o[6] | ((uint32_t)o[7] << 16);
      b.x = o[8] | ((uint32_t)o[9] << 16); b.y = o[10] | ((uint32_t)o[11] << 16);
      b.z = o[12] | ((uint32_t)o[13] << 16); b.w = o[14] | ((uint32_t)o[15] << 16);
      *(uint4*)dst = a;
      *(uint4*)(dst + 8) = b;
    }
    return;  // uniform per workgroup
  }
#pragma unroll
  for (int e = 0; e < 16; e++) vt[tl][c0 + e] = v[e];
  __syncthreads();
  // V^T[hk][d][L + t]: lane = token, so one store instruction writes
  // contiguous positions of two dimension rows (of one sequence, unless
  // the 32 tokens straddle two)
  const int hk = (cb * 128 - ea.qdim - ea.kvdim) >> 7;
  const int tt = tid & 31, dg = tid >> 5;
  const int tw = blockIdx.y * RQ_TOK + tt;
  if (tw < M) {
    const int bw = tw / ea.rps, tlw = tw - bw * ea.rps;
    uint16_t* base = (uint16_t*)ea.vt_cache + bw * ea.kv_seq + (size_t)hk * 128 * ea.max_ctx +
                     ea.st[bw].L + tlw;
#pragma unroll
    for (int e = 0; e < 16; e++) {
      const int d = dg * 16 + e;
      base[(size_t)d * ea.max_ctx] = f2bf(vt[tt][d]);
    }
  }
}

__device__ inline float block_sum(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); i++) t += sh[i];
  __syncthreads();
  return t;
}

// residual add; the next GEMM's input bf16(x * w) in fragment layout
// (deferred RMSNorm) and this chunk's sum of squares.  Workgroup (c, t):
// columns c*SSQ_CHUNK .. +SSQ_CHUNK of row t, 8 per thread.
// KS > 0: that many splits, every partial loaded before the first add (one
// memory round trip); KS == 0: ks splits, loaded one after another.  The
// splits are added in order either way.
template <int KS>
__global__ __launch_bounds__(SSQ_CHUNK / 8) void k_red_resid_scale(
    const float* __restrict__ P, int ks, int d, int M, float* __restrict__ x,
    const uint16_t* __restrict__ w, uint16_t* __restrict__ xnf, int MTT, float* __restrict__ ssq) {
  __shared__ float sh[SSQ_CHUNK / 8 / 64];
  const int c = blockIdx.x, t = blockIdx.y;
  const int i = c * SSQ_CHUNK + threadIdx.x * 8;
  float ss = 0.f;
  if (i < d) {
    float* xr = x + (size_t)t * d;
    const uint4 wv = *(const uint4*)(w + i);
    float v[8];
    load8(xr + i, v);
    if constexpr (KS > 0) {
      float p[KS][8];
#pragma unroll
      for (int z = 0; z < KS; z++) load8(P + ((size_t)z * M + t) * d + i, p[z]);
#pragma unroll
      for (int z = 0; z < KS; z++)
#pragma unroll
        for (int e = 0; e < 8; e++) v[e] += p[z][e];
    } else {
      for (int z = 0; z < ks; z++) {
        float p[8];
        load8(P + ((size_t)z * M + t) * d + i, p);
#pragma unroll
        for (int e = 0; e < 8; e++) v[e] += p[e];
      }
    }
    *(float4*)(xr + i) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(xr + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    const uint32_t wb[4] = {wv.x, wv.y, wv.z, wv.w};
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      ss = fmaf(v[e], v[e], ss);
      o[e] = v[e] * bf2f((uint16_t)(wb[e >> 1] >> ((e & 1) * 16)));
    }
    *(uint4*)&xnf[frag_index(t, i, MTT)] = pack8(o);
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
    for (int q = 0; q < SSQ_CHUNK / 8 / 64; q++) tot += sh[q];
    ssq[t * SSQ_STRIDE + c] = tot;
  }
}

// residual add + RMSNorm of the new row into fragment-layout bf16; one
// workgroup of 512 threads per row, 8 columns per thread per pass (up to
// two passes: d <= 8192); the row stays in registers between the sum of
// squares and the scaling
__global__ __launch_bounds__(512) void k_red_resid_norm(const float* __restrict__ P, int ks,
                                                        int d, int M, float* __restrict__ x,
                                                        const uint16_t* __restrict__ w,
                                                        float eps, uint16_t* __restrict__ xnf,
                                                        int MTT) {
  __shared__ float sh[8];
  const int t = blockIdx.x;
  float* xr = x + (size_t)t * d;
  float v[2][8];
  uint4 wv[2];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < 2; it++) {
    const int i = (it * 512 + threadIdx.x) * 8;
    if (i >= d) continue;
    wv[it] = *(const uint4*)(w + i);
    load8(xr + i, v[it]);
    for (int z = 0; z < ks; z++) {
      float p[8];
      load8(P + ((size_t)z * M + t) * d + i, p);
#pragma unroll
      for (int e = 0; e < 8; e++) v[it][e] += p[e];
    }
    *(float4*)(xr + i) = make_float4(v[it][0], v[it][1], v[it][2], v[it][3]);
    *(float4*)(xr + i + 4) = make_float4(v[it][4], v[it][5], v[it][6], v[it][7]);
#pragma unroll
    for (int e = 0; e < 8; e++) ss = fmaf(v[it][e], v[it][e], ss);
  }
  ss = block_sum(ss, sh);
  const float inv = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int it = 0; it < 2; it++) {
    const int i = (it * 512 + threadIdx.x) * 8;
    if (i >= d) continue;
    const uint32_t wb[4] = {wv[it].x, wv[it].y, wv[it].z, wv[it].w};
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; e++)
      o[e] = v[it][e] * inv * bf2f((uint16_t)(wb[e >> 1] >> ((e & 1) * 16)));
    *(uint4*)&xnf[frag_index(t, i, MTT)] = pack8(o);
  }
}

void launch_red_qkv(const float* P, int ks, int N, int M, const EpiArgs& ea, hipStream_t s) {
  const dim3 grid(N / 128, (M + RQ_TOK - 1) / RQ_TOK);
  if (ks == 1) hipLaunchKernelGGL(k_red_qkv<1>, grid, dim3(256), 0, s, P, ks, N, M, ea);
  else if (ks == 2) hipLaunchKernelGGL(k_red_qkv<2>, grid, dim3(256), 0, s, P, ks, N, M, ea);
  else if (ks == 4) hipLaunchKernelGGL(k_red_qkv<4>, grid, dim3(256), 0, s, P, ks, N, M, ea);
  else hipLaunchKernelGGL(k_red_qkv<0>, grid, dim3(256), 0, s, P, ks, N, M, ea);
}
void launch_red_resid_scale(const float* P, int ks, int d, int M, float* x, const uint16_t* w,
                            uint16_t* xnf, int MTT, float* ssq, hipStream_t s) {
  const dim3 grid((d + SSQ_CHUNK - 1) / SSQ_CHUNK, M), block(SSQ_CHUNK / 8);
#define LA_RED_CASE(k)                                                                              \
  case k:                                                                                           \
    hipLaunchKernelGGL(k_red_resid_scale<k>, grid, block, 0, s, P, ks, d, M, x, w, xnf, MTT, ssq); \
    break;
  switch (ks) {
    LA_RED_CASE(1)
    LA_RED_CASE(2)
    LA_RED_CASE(4)
    LA_RED_CASE(8)
    default:
      hipLaunchKernelGGL(k_red_resid_scale<0>, grid, block, 0, s, P, ks, d, M, x, w, xnf, MTT, ssq);
  }
#undef LA_RED_CASE
}
void launch_red_resid_norm(const float* P, int ks, int d, int M, float* x, const uint16_t* w,
                           float eps, uint16_t* xnf, int MTT, hipStream_t s) {
  hipLaunchKernelGGL(k_red_resid_norm, dim3(M), dim3(512), 0, s, P, ks, d, M, x, w, eps, xnf, MTT);
}

// ---------------------------------------------------------------------------
// One-tile GEMMs: at most 16 rows (one-token decode, small batches, small
// lookahead blocks).  The activations of a k-step are then one token tile
// of which only the valid rows' lanes are loaded (M x 64 bytes against the
// 1 KiB weight tile), so a workgroup can own a single 16-row weight tile
// over all of K and still stream nearly pure weights: 256 - 2000
// workgroups per GEMM without splitting K across workgroups.  The 8 waves
// of a workgroup take consecutive k ranges, each issuing V_U k-steps of
// loads before their MFMAs; their accumulators are summed through LDS in
// wave order (deterministic) and wave 0 applies the epilogue, so there are
// no fp32 partial sums in memory and no reduce kernel.  The deferred
// RMSNorm's row scale (QKV, gate/up inputs) comes from partial sums of
// squares that the producing epilogue wrote per 16 columns (or per 1024
// columns for the first layer's input), added in a fixed order.
constexpr int V_NW = 8;  // waves per workgroup
constexpr int V_U = 8;   // k-steps of loads per wave in flight

// sum over the lanes l, l^16, l^32, l^48 (same token column of a tile)
__device__ inline float sum_groups(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

template <int EPI>
__global__ __launch_bounds__(V_NW * 64) void k_gemv_bf16(GemvArgs a) {
  constexpr int NT = EPI == EPI_SWIGLU ? 2 : 1;  // weight tiles per workgroup
  __shared__ f32x4 red[V_NW][NT][64];
  __shared__ float invs[16];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wt = blockIdx.x;
  const int KS = a.K >> 5;
  const int k0 = KS * w / V_NW, k1 = KS * (w + 1) / V_NW;
  const int M = a.M;
  const bool live = (l & 15) < M;  // this lane's token column holds a row
  // weight tile wt (SWIGLU: gate tile 2 wt and up tile 2 wt + 1)
  const uint16_t* wb = a.Wp + (size_t)wt * NT * KS * 512 + l * 8;
  const uint16_t* xb = a.X + l * 8;

  if constexpr (EPI == EPI_QKV || EPI == EPI_SWIGLU) {
    // the input rows' 1/rms, tokens w and w + 8; its loads go out ahead
    // of the weight stream
    for (int t = w; t < M; t += V_NW) {
      float sq = 0.f;
      for (int i = l; i < a.ssq_n; i += 64) sq += a.ssq[(size_t)t * a.ssq_stride + i];
      for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o);
      if (l == 0) invs[t] = 1.f / sqrtf(sq / (float)a.d_in + a.eps);
    }
  }

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; j++) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int ks = k0;
  for (; ks + V_U <= k1; ks += V_U) {
    bf16x8 wv[NT][V_U], xv[V_U];
#pragma unroll
    for (int u = 0; u < V_U; u++)
#pragma unroll
      for (int j = 0; j < NT; j++)
        wv[j][u] = __builtin_nontemporal_load((const bf16x8*)(wb + ((size_t)j * KS + ks + u) * 512));
#pragma unroll
    for (int u = 0; u < V_U; u++) xv[u] = bf16x8{};
    if (live) {
#pragma unroll
      for (int u = 0; u < V_U; u++) xv[u] = *(const bf16x8*)(xb + (size_t)(ks + u) * a.MTT * 512);
    }
#pragma unroll
    for (int u = 0; u < V_U; u++)
#pragma unroll
      for (int j = 0; j < NT; j++)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[j][u], xv[u], acc[j], 0, 0, 0);
  }
  for (; ks < k1; ks++) {
    bf16x8 wv[NT], xv = bf16x8{};
#pragma unroll
    for (int j = 0; j < NT; j++)
      wv[j] = __builtin_nontemporal_load((const bf16x8*)(wb + ((size_t)j * KS + ks) * 512));
    if (live) xv = *(const bf16x8*)(xb + (size_t)ks * a.MTT * 512);
#pragma unroll
    for (int j = 0; j < NT; j++)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[j], xv, acc[j], 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < NT; j++) red[w][j][l] = acc[j];
  __syncthreads();
  if (w != 0) return;

  // lane l: output rows n = 16 wt + 4 g + i (i = 0..3) of token t
  f32x4 sum[NT];
#pragma unroll
  for (int j = 0; j < NT; j++) {
    sum[j] = red[0][j][l];
#pragma unroll
    for (int ww = 1; ww < V_NW; ww++) sum[j] += red[ww][j][l];
  }
  const int t = l & 15, g = l >> 4;
  const int n = wt * 16 + 4 * g;

  if constexpr (EPI == EPI_LOGITS) {
    if (t < M) *(f32x4*)&a.logits[(size_t)t * a.N + n] = sum[0];
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (t < M) {
      const float inv = invs[t];
      const f32x4 gt = sum[0] * inv, u = sum[1] * inv;
      uint2 pk;
      pk.x = (uint32_t)f2bf(silu(gt[0]) * u[0]) | ((uint32_t)f2bf(silu(gt[1]) * u[1]) << 16);
      pk.y = (uint32_t)f2bf(silu(gt[2]) * u[2]) | ((uint32_t)f2bf(silu(gt[3]) * u[3]) << 16);
      *(uint2*)&a.act[frag_index(t, n, a.MTT)] = pk;
    }
  } else if constexpr (EPI == EPI_RESID) {
    float ss = 0.f;
    if (t < M) {
      float* xr = a.x + (size_t)t * a.N + n;
      const f32x4 v = *(const f32x4*)xr + sum[0];
      *(f32x4*)xr = v;
      if (a.xnf) {
        const uint2 wv = *(const uint2*)(a.wn + n);
        uint2 pk;
        pk.x = (uint32_t)f2bf(v[0] * bf2f((uint16_t)wv.x)) | ((uint32_t)f2bf(v[1] * bf2f((uint16_t)(wv.x >> 16))) << 16);
        pk.y = (uint32_t)f2bf(v[2] * bf2f((uint16_t)wv.y)) | ((uint32_t)f2bf(v[3] * bf2f((uint16_t)(wv.y >> 16))) << 16);
        *(uint2*)&a.xnf[frag_index(t, n, a.MTT)] = pk;
      }
      ss = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], v[3] * v[3])));
    }
    ss = sum_groups(ss);
    if (g == 0 && t < M) a.ssq_out[(size_t)t * (a.N >> 4) + wt] = ss;
  } else {  // EPI_QKV: 1/rms, RoPE on q and k, q rows and the KV cache
    if (t < M) {
      const EpiArgs& ea = a.ea;
      const f32x4 v = sum[0] * invs[t];
      const int b = t / ea.rps, tl = t - b * ea.rps;
      const int L = ea.st[b].L;
      if (n < ea.qdim + ea.kvdim) {
        const int di = (n < ea.qdim ? n : n - ea.qdim) & 127;  // dim within the head
        const float* cs = ea.rope_rows + (size_t)t * 128 + di / 2;
        const float c0 = cs[0], c1 = cs[1], s0 = cs[64], s1 = cs[65];
        uint2 pk;
        pk.x = (uint32_t)f2bf(v[0] * c0 - v[1] * s0) | ((uint32_t)f2bf(v[0] * s0 + v[1] * c0) << 16);
        pk.y = (uint32_t)f2bf(v[2] * c1 - v[3] * s1) | ((uint32_t)f2bf(v[2] * s1 + v[3] * c1) << 16);
        uint16_t* dst;
        if (n < ea.qdim) {
          dst = (uint16_t*)ea.out_act + (size_t)t * ea.qdim + n;
        } else {
          const int hk = (n - ea.qdim) >> 7;
          dst = (uint16_t*)ea.k_cache + b * ea.kv_seq + ((size_t)hk * ea.max_ctx + L + tl) * 128 + di;
        }
        *(uint2*)dst = pk;
      } else {
        const int vv = n - ea.qdim - ea.kvdim, hk = vv >> 7, di = vv & 127;
        uint16_t* dst = (uint16_t*)ea.vt_cache + b * ea.kv_seq + ((size_t)hk * 128 + di) * ea.max_ctx + L + tl;
#pragma unroll
        for (int i = 0; i < 4; i++) dst[(size_t)i * ea.max_ctx] = f2bf(v[i]);
      }
    }
  }
}

bool gemv_bf16_ok(int M, int N, int K) { return M >= 1 && M <= 16 && N % 32 == 0 && K % 32 == 0; }

void launch_gemv_bf16(int epi, const GemvArgs& a, hipStream_t s) {
  const dim3 block(V_NW * 64);
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL(k_gemv_bf16<EPI_QKV>, dim3(a.N / 16), block, 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL(k_gemv_bf16<EPI_RESID>, dim3(a.N / 16), block, 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemv_bf16<EPI_SWIGLU>, dim3(a.N / 32), block, 0, s, a); break;
    default: hipLaunchKernelGGL(k_gemv_bf16<EPI_LOGITS>, dim3(a.N / 16), block, 0, s, a); break;
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

void launch_repack_bf16(const uint16_t* src, int rows, int K, uint16_t* dst, int rt_offset,
                        int rt_mult, hipStream_t s) {
  size_t lanes = (size_t)(rows / 16) * (K / 32) * 64;
  int blocks = (int)((lanes + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_repack_bf16, dim3(blocks), dim3(256), 0, s, src, rows, K, dst, rt_offset,
                     rt_mult);
}

// ---------------------------------------------------------------------------
// fp32 kernel (small models): one thread per (row, output pair), direct
// epilogues on row-major activations

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
    float* o = (float*)ea.out_act + (size_t)t * ea.ld_out + n;
    o[0] = silu(s0) * u0;
    o[1] = silu(s1) * u1;
  } else if (EPI == EPI_QKV) {
    qkv_pair<float>(ea, t, n, s0, s1);
  } else if (EPI == EPI_RESID) {
    float* o = ea.out_f32 + (size_t)t * ea.ld_out + n;
    o[0] += s0;
    o[1] += s1;
  } else {
    float* o = ea.out_f32 + (size_t)t * ea.ld_out + n;
    o[0] = s0;
    o[1] = s1;
  }
}

void launch_gemm_f32(int epi, const float* X, const float* W, const float* W2, int K, int N,
                     int M, const EpiArgs& ea, hipStream_t s) {
  dim3 grid((N / 2 + 63) / 64, M), block(64);
  switch (epi) {
    case EPI_LOGITS: hipLaunchKernelGGL(k_gemm_f32<EPI_LOGITS>, grid, block, 0, s, X, W, W2, K, N, M, ea); break;
    case EPI_RESID: hipLaunchKernelGGL(k_gemm_f32<EPI_RESID>, grid, block, 0, s, X, W, W2, K, N, M, ea); break;
    case EPI_QKV: hipLaunchKernelGGL(k_gemm_f32<EPI_QKV>, grid, block, 0, s, X, W, W2, K, N, M, ea); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_f32<EPI_SWIGLU>, grid, block, 0, s, X, W, W2, K, N, M, ea); break;
  }
}

}  // namespace la
