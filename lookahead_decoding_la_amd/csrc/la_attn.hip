// Masked attention of the lookahead step: every block row attends to the
// whole committed cache and to the block rows the lookahead/verification
// mask lets it see ("Break the Sequential Dependency of LLM Inference Using
// Lookahead Decoding", Summary: lookahead and verification branches share
// one forward pass; the method works with FlashAttention-style kernels).
//
// bf16 kernel (gfx950, head_dim 128):
//   - grid = heads x 64-row token groups x KV splits (flash-decoding style
//     split of the key range so short contexts still fill 256 CUs);
//   - each 64-key chunk of K and of V^T is staged once in LDS (padded rows,
//     no bank conflicts) and shared by the 4 waves of the workgroup;
//   - S^T = K Q^T on MFMA, so a lane owns one token's scores; the mask is
//     computed from (row, key) indices, never loaded; the online softmax
//     max/sum are wave-level reductions across the 4 lane groups;
//   - O^T = V^T P^T on MFMA: P^T feeds MFMA straight from the score
//     registers (the 32 keys of one k-step are taken in the order the score
//     layout holds them, V^T is read in the same order);
//   - splits merge in a second kernel (log-sum-exp weights).
// The cache stores V transposed ([kv head][dh][position]) for this reason.
#include "la_epilogue.h"

namespace la {

constexpr int AKC = 64;       // keys per chunk
constexpr int A_DH = 128;     // head_dim of the bf16 kernel
constexpr int KPAD = A_DH + 8;  // LDS row stride of K (elements)
constexpr int VPAD = AKC + 8;   // LDS row stride of V^T (elements)
constexpr float LOG2E = 1.4426950408889634f;

__device__ inline float wave_max_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ inline float wave_sum_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ inline bool key_visible(int mode, const RowDesc& rd, int t, int M,
                                   int L, int p, int W, int N) {
  if (p < L) return true;
  const int b = p - L;
  if (b >= M) return false;
  if (t >= M) return true;  // padding rows: anything finite
  if (mode == MODE_CAUSAL) return b <= t;
  return row_sees(rd, row_desc(b, W, N));
}

__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a) {
  __shared__ uint16_t Ks[AKC * KPAD];
  __shared__ uint16_t Vs[A_DH * VPAD];

  const int h = blockIdx.x, tg = blockIdx.y, sp = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;
  const int L = a.st ? a.st->L : a.L_host;
  const int M = a.M;
  const int kvh = (h * a.Hkv) / a.H;
  const int ctx = L + M;
  const int nch = (ctx + AKC - 1) / AKC;
  const int cps = (nch + a.splits - 1) / a.splits;
  const int c0 = sp * cps, c1 = min(nch, c0 + cps);
  const int t0 = tg * 64 + w * 16;
  const bool active = t0 < M;
  const int t = t0 + c16;
  const int rows16 = (M + 15) & ~15;
  const RowDesc rd = row_desc(t < M ? t : 0, a.W, a.N);
  const float sl2 = LOG2E / sqrtf((float)A_DH);

  const uint16_t* kc = (const uint16_t*)a.k_cache + (size_t)kvh * a.ctx_stride * A_DH;
  const uint16_t* vc = (const uint16_t*)a.vt_cache + (size_t)kvh * A_DH * a.ctx_stride;

  bf16x8 qf[4];
  if (t < M) {
    const uint16_t* qrow = (const uint16_t*)a.q + (size_t)t * (a.H * A_DH) + h * A_DH;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) qf[ks] = *(const bf16x8*)(qrow + ks * 32 + g * 8);
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
#pragma unroll
      for (int e = 0; e < 8; e++) qf[ks][e] = (__bf16)0.f;
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; i++) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = c0; c < c1; c++) {
    __syncthreads();
    // stage K [64 keys][128] and V^T [128][64 keys]; chunk c lies inside the
    // cache allocation because ctx <= max_ctx <= ctx_stride (a multiple of 64)
#pragma unroll
    for (int i = tid; i < AKC * A_DH / 8; i += 256) {
      const int r = i >> 4, cv = i & 15;
      const uint4 v = *(const uint4*)(kc + (size_t)(c * AKC + r) * A_DH + cv * 8);
      *(uint4*)&Ks[r * KPAD + cv * 8] = v;
    }
#pragma unroll
    for (int i = tid; i < A_DH * AKC / 8; i += 256) {
      const int dr = i >> 3, cv = i & 7;
      const uint4 v = *(const uint4*)(vc + (size_t)dr * a.ctx_stride + c * AKC + cv * 8);
      *(uint4*)&Vs[dr * VPAD + cv * 8] = v;
    }
    __syncthreads();
    if (!active) continue;

    // scores: s[kt][v] = key c*64 + kt*16 + 4g + v, token c16
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        const bf16x8 kf = *(const bf16x8*)&Ks[(kt * 16 + c16) * KPAD + ks * 32 + g * 8];
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[kt], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
    const bool full = (c + 1) * AKC <= L;  // whole chunk in the committed prefix
#pragma unroll
    for (int kt = 0; kt < 4; kt++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        float x = s[kt][v] * sl2;
        if (!full) {
          const int p = c * AKC + kt * 16 + 4 * g + v;
          if (!key_visible(a.mode, rd, t, M, L, p, a.W, a.N)) x = -INFINITY;
        }
        s[kt][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = wave_max_groups(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; kt++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const float p = (m_new == -INFINITY) ? 0.f : exp2f(s[kt][v] - m_new);
        s[kt][v] = p;
        ps += p;
      }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] *= alpha;
    m_run = m_new;

#pragma unroll
    for (int s2 = 0; s2 < 2; s2++) {
      bf16x8 pf;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        pf[v] = (__bf16)s[2 * s2][v];
        pf[4 + v] = (__bf16)s[2 * s2 + 1][v];
      }
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const uint16_t* vr = &Vs[(dt * 16 + c16) * VPAD + 32 * s2 + 4 * g];
        const uint2 lo = *(const uint2*)vr;
        const uint2 hi = *(const uint2*)(vr + 16);
        bf16x8 vf;
        uint4 pack = {lo.x, lo.y, hi.x, hi.y};
        vf = *(bf16x8*)&pack;
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[dt], 0, 0, 0);
      }
    }
  }

  if (!active) return;
  l_run = wave_sum_groups(l_run);
  if (t >= M) return;
  if (a.splits == 1) {
    // row-major, or fragment layout (dims dt*16 + 4g + 0..3 stay adjacent)
    uint16_t* out = (uint16_t*)a.out;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      const int k = h * A_DH + dt * 16 + 4 * g;
      const size_t o0 = a.out_mtt ? frag_index(t, k, a.out_mtt) : (size_t)t * (a.H * A_DH) + k;
#pragma unroll
      for (int v = 0; v < 4; v++) out[o0 + v] = f2bf(o[dt][v] * inv);
    }
  } else {
    float* po = a.part_o + (((size_t)h * a.splits + sp) * rows16 + t) * A_DH;
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      *(f32x4*)&po[dt * 16 + 4 * g] = o[dt];
    if (g == 0) {
      float* pm = a.part_ml + (((size_t)h * a.splits + sp) * rows16 + t) * 2;
      pm[0] = m_run;
      pm[1] = l_run;
    }
  }
}

// combine the splits of one (row, head): weights 2^(m_s - m*)
__global__ void k_attn_merge(AttnArgs a) {
  const int t = blockIdx.x, h = blockIdx.y, i = threadIdx.x;  // i < dh
  const int rows16 = (a.M + 15) & ~15;
  float mstar = -INFINITY;
  for (int s = 0; s < a.splits; s++)
    mstar = fmaxf(mstar, a.part_ml[(((size_t)h * a.splits + s) * rows16 + t) * 2]);
  float den = 0.f, num = 0.f;
  for (int s = 0; s < a.splits; s++) {
    const size_t b = ((size_t)h * a.splits + s) * rows16 + t;
    const float m = a.part_ml[b * 2];
    const float wgt = (m == -INFINITY) ? 0.f : exp2f(m - mstar);
    den += wgt * a.part_ml[b * 2 + 1];
    num += wgt * a.part_o[b * A_DH + i];
  }
  const int k = h * A_DH + i;
  const size_t o = a.out_mtt ? frag_index(t, k, a.out_mtt) : (size_t)t * (a.H * A_DH) + k;
  ((uint16_t*)a.out)[o] = f2bf(num / den);
}

int attn_bf16_splits(int H, int M, int max_ctx) {
  const int tgs = (M + 63) / 64;
  const int max_chunks = (max_ctx + AKC - 1) / AKC;
  int s = 1;
  while (H * tgs * s < 512 && s * 2 <= max_chunks && s < 64) s *= 2;
  return s;
}

size_t attn_bf16_partial_floats(int H, int M, int splits, int dh) {
  const int rows16 = (M + 15) & ~15;
  return (size_t)H * splits * rows16 * (dh + 2);
}

void launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.H, (a.M + 63) / 64, a.splits);
  hipLaunchKernelGGL(k_attn_bf16, grid, dim3(256), 0, s, a);
  if (a.splits > 1)
    hipLaunchKernelGGL(k_attn_merge, dim3(a.M, a.H), dim3(A_DH), 0, s, a);
}

// ---------------------------------------------------------------------------
// fp32 kernel (small models, head_dim <= 256): one wave per (row, head),
// scores for every key in LDS, exact softmax.

__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
  extern __shared__ float sc[];
  const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int L = a.st ? a.st->L : a.L_host;
  const int M = a.M, dh = a.dh;
  const int kvh = (h * a.Hkv) / a.H;
  const int ctx = L + M;
  const float* q = (const float*)a.q + (size_t)t * a.H * dh + (size_t)h * dh;
  const float* kc = (const float*)a.k_cache + (size_t)kvh * a.ctx_stride * dh;
  const float* vc = (const float*)a.vt_cache + (size_t)kvh * dh * a.ctx_stride;
  const RowDesc rd = row_desc(t, a.W, a.N);
  const float scale = 1.f / sqrtf((float)dh);
  float mx = -INFINITY;
  for (int j = tid; j < ctx; j += 64) {
    float s = -INFINITY;
    if (key_visible(a.mode, rd, t, M, L, j, a.W, a.N)) {
      const float* k = kc + (size_t)j * dh;
      float acc = 0.f;
      for (int i = 0; i < dh; i++) acc = fmaf(q[i], k[i], acc);
      s = acc * scale;
    }
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float z = 0.f;
  for (int j = tid; j < ctx; j += 64) {
    const float e = sc[j] == -INFINITY ? 0.f : expf(sc[j] - mx);
    sc[j] = e;
    z += e;
  }
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  __syncthreads();
  float* out = (float*)a.out + (size_t)t * a.H * dh + (size_t)h * dh;
  for (int i = tid; i < dh; i += 64) {
    const float* v = vc + (size_t)i * a.ctx_stride;
    float acc = 0.f;
    for (int j = 0; j < ctx; j++) acc = fmaf(sc[j], v[j], acc);
    out[i] = acc / z;
  }
}

void launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_attn_f32, dim3(a.M, a.H), dim3(64), sizeof(float) * a.ctx_stride, s, a);
}

}  // namespace la
