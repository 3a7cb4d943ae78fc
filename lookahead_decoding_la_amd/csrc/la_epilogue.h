// Output-side helpers of the GEMMs and their epilogues: the MFMA fragment
// layout of bf16 activations, SiLU, and the fp32 GEMM's fused-QKV epilogue
// (RoPE + q / KV-cache stores).
#pragma once

#include "la_internal.h"

namespace la {

// bf16 activations that feed a GEMM are stored in the MFMA B-operand
// fragment layout: for k-step ks (32 columns) and token tile m (16 rows)
// one 1 KiB block of 64 lanes x 8 values, lane = 16*((k%32)/8) + t%16.
// MTT = token tiles of the buffer.  A GEMM wave then loads a whole B
// fragment as one contiguous 1 KiB read.
__host__ __device__ inline size_t frag_index(int t, int k, int MTT) {
  return ((((size_t)(k >> 5) * MTT + (t >> 4)) * 64 + ((k & 31) >> 3) * 16 + (t & 15)) << 3) +
         (k & 7);
}

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

__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

// Fused-QKV epilogue for the adjacent output columns (n, n+1), n even, of
// row t (block row tl = t % rps of sequence b = t / rps): q and k are
// rotated by angle pos * theta^(-2i/dh) (i = pair index within the head)
// at absolute position L_b + relpos[t] and stored; v goes to the
// transposed V cache.  The block row's key/value sit at cache position
// L_b + tl of its sequence.
template <typename ACT>
__device__ inline void qkv_pair(const EpiArgs& ea, int t, int n, float v0, float v1) {
  const int b = t / ea.rps, tl = t - b * ea.rps;
  const int L = ea.st[b].L;
  const int dh = ea.dh;
  if (n < ea.qdim + ea.kvdim) {
    const int di = (n < ea.qdim ? n : n - ea.qdim) % dh;
    const int pos = L + ea.relpos[t];
    const float c = ea.rope_cos[(size_t)pos * (dh / 2) + di / 2];
    const float s = ea.rope_sin[(size_t)pos * (dh / 2) + di / 2];
    const float r0 = v0 * c - v1 * s, r1 = v0 * s + v1 * c;
    if (n < ea.qdim) {
      const size_t o = (size_t)t * ea.qdim + n;
      store_act<ACT>(ea.out_act, o, r0);
      store_act<ACT>(ea.out_act, o + 1, r1);
    } else {
      const int hk = (n - ea.qdim) / dh;
      const size_t o = b * ea.kv_seq + ((size_t)hk * ea.max_ctx + L + tl) * dh + di;
      store_act<ACT>(ea.k_cache, o, r0);
      store_act<ACT>(ea.k_cache, o + 1, r1);
    }
  } else {
    const int vv = n - ea.qdim - ea.kvdim, hk = vv / dh, di = vv % dh;
    const size_t o = b * ea.kv_seq + ((size_t)hk * dh + di) * ea.max_ctx + L + tl;
    store_act<ACT>(ea.vt_cache, o, v0);
    store_act<ACT>(ea.vt_cache, o + ea.max_ctx, v1);
  }
}

}  // namespace la
