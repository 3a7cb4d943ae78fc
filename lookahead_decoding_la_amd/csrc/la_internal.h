// Internal declarations shared by the HIP sources of the lookahead library.
// Device helpers, the block-row mask, kernel parameter structs and the host
// launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// ---------------------------------------------------------------------------
// element types

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bfloat16 <-> float through bit patterns (round to nearest even).
__host__ __device__ inline float bf2f(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return v.f;
}
__host__ __device__ inline uint16_t f2bf(float f) {
  union { uint32_t u; float f; } v;
  v.f = f;
  uint32_t u = v.u;
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Waits and barriers for kernels that load through global_load_lds (LDS
// direct loads): the compiler does not order those loads against LDS reads
// of other waves, so the kernels wait on vmcnt themselves and then meet at
// a barrier.

// s_waitcnt with vmcnt(n), other counters untouched (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int n>
__device__ inline void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's LDS operations have completed
// (lgkmcnt(0)).  Unlike __syncthreads it does not wait for outstanding
// global loads, so the chunks in flight stay in flight.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Device-resident decoding state.  Scalars that change every step live here
// (not in launch arguments) so one captured graph replays every step.

struct DevState {
  int32_t L;       // committed KV length
  int32_t cur;     // current token (its KV is not committed yet)
  int32_t n_cand;  // valid candidates in the block being forwarded
  int32_t L_old;   // committed length before the last commit
  int32_t k;       // accepted candidate tokens of the last step
  int32_t winner;  // g* of the last step, -1 without candidates
  int32_t pad[2];
};

// Mirror of la_step_result (include/la.h); written by the verify kernel and
// copied to pinned host memory at the end of a step.
struct DevResult {
  int32_t n_emitted;
  int32_t tokens[32];
  int32_t accepted;
  int32_t winner;
  int32_t n_candidates;
  int32_t kv_len;
};

// Mask modes of a forwarded block.
enum { MODE_STEP = 0, MODE_CAUSAL = 1 };

// Per-sequence token selection: temperature 0 takes the argmax; otherwise
// the emitted tokens are draws (la_sample.hip).
struct SampleParams {
  float temperature;  // 0: argmax
  float top_p;        // (0, 1], 1: no cut
  int32_t top_k;      // 0: no cut
  uint32_t seed_lo, seed_hi;
  int32_t pad[3];
};
constexpr int SAMPLE_MAX_VOCAB = 32768;  // 1024 threads x 32 logits per row

// ---------------------------------------------------------------------------
// Block-row layout of one lookahead step ("Break the Sequential Dependency of
// LLM Inference Using Lookahead Decoding", Summary: the lookahead branch's 2D
// window and the verification branch run in one forward pass).
//   row 0                        current token, relative position 0
//   1 + (l-1)*W + j              window level l (1..N-1), column j;
//                                relative position l + j
//   1 + (N-1)*W + g*(N-1) + i-1  candidate g, token i (1..N-1); position i
// A row sees the whole committed cache plus: row 0 sees itself; window row
// (l, j) sees row 0, level-1 rows of columns <= j and the rows of column j at
// levels 2..l; candidate row (g, i) sees row 0 and (g, i') for i' <= i.  So
// each row sees exactly one causal sequence: its column's diagonal through
// the window, or its candidate's prefix.

struct RowDesc {
  int kind;  // 0 current, 1 window, 2 candidate
  int a, b;  // window: level (1-based), column; candidate: g, i (1-based)
};

__host__ __device__ inline RowDesc row_desc(int r, int W, int N) {
  RowDesc d;
  int nwin = (N - 1) * W;
  if (r == 0) { d.kind = 0; d.a = 0; d.b = 0; }
  else if (r <= nwin) { d.kind = 1; d.a = 1 + (r - 1) / W; d.b = (r - 1) % W; }
  else { d.kind = 2; d.a = (r - 1 - nwin) / (N - 1); d.b = 1 + (r - 1 - nwin) % (N - 1); }
  return d;
}

__host__ __device__ inline int row_relpos(const RowDesc& d) {
  return d.kind == 0 ? 0 : (d.kind == 1 ? d.a + d.b : d.b);
}

// Does the row described by q see block row described by k?
__host__ __device__ inline bool row_sees(const RowDesc& q, const RowDesc& k) {
  if (k.kind == 0) return true;
  if (q.kind != k.kind) return false;
  if (q.kind == 1) return k.a == 1 ? k.b <= q.b : (k.b == q.b && k.a <= q.a);
  return k.a == q.a && k.b <= q.b;
}

// ---------------------------------------------------------------------------
// launch parameters

struct ModelDims {
  int n_layers, d, H, Hkv, dh, ffn, V;
  int W, N, G;
  int max_ctx;
  float eps;
};

// GEMM epilogues.
enum { EPI_LOGITS = 0, EPI_RESID = 1, EPI_QKV = 2, EPI_SWIGLU = 3 };

// Batched rows: row t belongs to sequence t / rps (relative to the state
// and cache pointers, which point at the first sequence the launch covers)
// and is that sequence's block row t % rps.  Sequence b's caches start
// b * kv_seq elements after the pointers.
struct EpiArgs {
  int M;                 // valid rows
  float* out_f32;        // LOGITS: [M][N]; RESID: residual [M][N], added to
  void* out_act;         // SWIGLU: [M][ffn] activation; QKV: q [M][H*dh]
  void* k_cache;         // QKV: [seq][Hkv][max_ctx][dh] of this layer
  void* vt_cache;        // QKV: [seq][Hkv][dh][max_ctx] of this layer
  const DevState* st;    // QKV: committed length L, one state per sequence
  const int32_t* relpos; // QKV: relative position of each row
  int rps;               // QKV: rows per sequence
  size_t kv_seq;         // QKV: cache elements per sequence (Hkv*max_ctx*dh)
  const float* rope_cos; // [max_ctx][dh/2]
  const float* rope_sin;
  int qdim, kvdim, dh, max_ctx, ld_out;
  const float* rope_rows;  // bf16 QKV: per block row, cos[64] then sin[64] at
                           // the row's absolute position (written by assembly)
  const float* ssq;      // bf16 QKV: per-row partial sums of squares of the
  int ssn, dmodel;       //   un-normalized input [rows][8] (ssn used), so
  float eps;             //   outputs are scaled by the row's 1/rms here
};

// Deferred RMSNorm.  A GEMM input written as bf16(x * w) (norm weight w,
// without the row's 1/rms) gives outputs that the consumer scales by
// row_inv_rms: the row scale commutes with the product.  ssq[t][0..ssn)
// hold partial sums of x^2 over column chunks, summed in chunk order.
constexpr int SSQ_STRIDE = 8;
constexpr int SSQ_CHUNK = 1024;  // columns per partial sum
__device__ inline float row_inv_rms(const float* ssq, int ssn, int t, int d, float eps) {
  float s = 0.f;
  for (int i = 0; i < ssn; i++) s += ssq[t * SSQ_STRIDE + i];
  return 1.f / sqrtf(s / (float)d + eps);
}

// ---------------------------------------------------------------------------
// host launchers (one per kernel family)

// bf16 weights repacked into MFMA A-operand tiles (16 rows x 32 k, 1 KiB):
// tile (rt, ks) at element offset (rt * (K/32) + ks) * 512; lane l holds
// W[rt*16 + l%16][ks*32 + (l/16)*8 + e], e = 0..7.
void launch_repack_bf16(const uint16_t* src, int rows, int K, uint16_t* dst,
                        int rt_offset, int rt_mult, hipStream_t s);

// bf16 GEMM: P[z][t][n] (fp32, row stride N) = partial sum over the z-th
// K split of X[t][:] W[n][:]; X in fragment layout with MTT token tiles.
struct GemmPlan {
  int ksplit;  // K splits (workgroups per 128-row tile)
  int J;       // k-steps per pipeline stage
};
GemmPlan gemm_bf16_plan(int N, int K, int rows);
void launch_gemm_bf16(const uint16_t* X, int MTT, const uint16_t* Wp, int K, int N, int M,
                      const GemmPlan& plan, float* P, hipStream_t s);
// Fused gate/up (alternating 16-row gate / up tiles, no K split) with the
// SwiGLU written to fragment-layout A (FFN width N/2).
void launch_gemm_bf16_swiglu(const uint16_t* X, int MTT, const uint16_t* Wp, int K, int N, int M,
                             int J, uint16_t* A, const float* ssq, int ssn, float eps,
                             hipStream_t s);
// One-tile GEMMs (at most 16 rows: one token tile): a workgroup owns one
// 16-row weight tile (QKV, O, down, LM head) or one gate/up tile pair over
// all of K, splits K over its waves, sums them through LDS in wave order
// and applies the epilogue itself (no partial sums in memory).
struct GemvArgs {
  const uint16_t* X;  // input in fragment layout (token tile 0 of each k-step)
  int MTT;            // token tiles per k-step of X (and of xnf / act)
  const uint16_t* Wp; // packed weight tiles
  int K, N, M;        // reduction length, output rows, valid tokens (1..16)
  // QKV, SWIGLU: deferred RMSNorm of the input rows: partial sums of
  // squares ssq[t * ssq_stride + i], i < ssq_n, over d_in columns
  const float* ssq;
  int ssq_n, ssq_stride, d_in;
  float eps;
  // RESID (O, down): x [M][N] += Y; bf16(x * wn) into xnf (fragment layout,
  // skipped when xnf is NULL) and each 16-column tile's sum of squares of
  // the new x into ssq_out[t * (N / 16) + tile]
  float* x;
  const uint16_t* wn;
  uint16_t* xnf;
  float* ssq_out;
  uint16_t* act;   // SWIGLU: FFN activation (N / 2 wide), fragment layout
  float* logits;   // LOGITS: [M][N]
  EpiArgs ea;      // QKV: q rows, the caches, rotary factors per row
};
bool gemv_bf16_ok(int M, int N, int K);
void launch_gemv_bf16(int epi, const GemvArgs& a, hipStream_t s);

// reduce kernels (sum K splits in order + epilogue)
void launch_red_qkv(const float* P, int ks, int N, int M, const EpiArgs& ea, hipStream_t s);
// residual add; next GEMM input bf16(x * w) in fragment layout and the
// row's partial sums of squares (deferred RMSNorm), one workgroup per
// SSQ_CHUNK columns of a row
void launch_red_resid_scale(const float* P, int ks, int d, int M, float* x, const uint16_t* w,
                            uint16_t* xnf, int MTT, float* ssq, hipStream_t s);
void launch_red_resid_norm(const float* P, int ks, int d, int M, float* x, const uint16_t* w,
                           float eps, uint16_t* xnf, int MTT, hipStream_t s);

// fp32 path (small models): Y = X W^T with W row-major [N][K] (two
// matrices for SWIGLU: W2 is the up projection).
void launch_gemm_f32(int epi, const float* X, const float* W, const float* W2,
                     int K, int N, int M, const EpiArgs& ea, hipStream_t s);

// masked attention over the cache + block
// Batched: sequence b (grid z) owns rows b*rps .. b*rps + M - 1 of q and
// out, state st[b] and the caches b * kv_seq elements on.
struct AttnArgs {
  const void* q;       // [rows][H*dh] (bf16 or f32)
  const void* k_cache; // [seq][Hkv][ctx_stride][dh]
  const void* vt_cache;// [seq][Hkv][dh][ctx_stride]
  void* out;           // f32: [rows][H*dh]; bf16: fragment layout, MTT tiles
  int out_mtt;
  const DevState* st;  // committed length L (device, per sequence), or NULL: use L_host
  int L_host;
  int M;               // rows of one sequence's block
  int rps, nseq;       // row stride between sequences, sequences
  size_t kv_seq;       // cache elements per sequence
  int mode;            // MODE_STEP / MODE_CAUSAL
  int H, Hkv, dh, ctx_stride, W, N;
  float* part_o;       // split-KV partials [seq][H][splits][rows16][dh]
  float* part_ml;      // [seq][H][splits][rows16][2]
  int splits;
  int vt_finite;       // 1: every V^T entry of the cache rows holds a finite value (the
                       // engine's caches), so the entries past the context in the last
                       // chunk need no zeroing; 0: they may hold anything
};
void launch_attn_bf16(const AttnArgs& a, hipStream_t s);
// whether launch_attn_bf16 takes the unsplit per-tile kernel (no partials)
bool attn_bf16_tiled(int M, int ctx_stride, int H, int nseq);
int attn_bf16_splits(int H, int M, int max_ctx);
void launch_attn_f32(const AttnArgs& a, hipStream_t s);

// small kernels
void launch_fill_u32(void* p, uint32_t v, size_t n, hipStream_t s);
// Also writes the first layer's normalized input: bf16 -> fragment layout
// (xnf, MTT tiles, norm weight nw); f32 -> nothing (a separate RMSNorm).
// Step mode: M = nseq * T rows, sequence b's state st[b], window
// win + b*(N-1)*W and pool pool_len + b*V, pool + b*V*G*(N-1).  Causal
// mode: one sequence (st, the prompt rows).
void launch_assemble(int mode, const DevState* st, const int32_t* win,
                     const int32_t* pool_len, const int32_t* pool,
                     const int32_t* prompt, int M, int T, int V, int W, int N, int G,
                     int32_t* tokens, int32_t* relpos, DevState* st_w,
                     const void* emb, int d, int bf16, float* x,
                     const uint16_t* nw, float eps, uint16_t* xnf, int MTT,
                     float* ssq, const float* rope_cos, const float* rope_sin,
                     float* rope_rows, hipStream_t s);
void launch_rmsnorm(const float* x, const void* w, int M, int d, float eps,
                    int bf16, void* out, hipStream_t s);
// The decision of each row (la_sample.hip): step mode (rows b*T.., state
// st[b], parameters sp[b]): lookahead rows and empty candidate slots take
// the argmax, the current-token and candidate rows a draw when sampling is
// on; causal mode (one sequence): row M-1 as the current-token row, the
// others the argmax.  A draw for the token at position L + relpos + 1.
void launch_select(const float* logits, int M, int V, int T, int mode, int W, int N,
                   const DevState* st, const int32_t* relpos, const SampleParams* sp,
                   int32_t* out, hipStream_t s);
// Draws from rows of logits with one parameter set, row r with the uniform
// of position positions[r].
void launch_sample_rows(const float* logits, int rows, int V, const SampleParams& p,
                        const int64_t* positions, int32_t* out, hipStream_t s);
// one workgroup per sequence (rows b*T.., window, pool and result b)
void launch_verify(DevState* st, const int32_t* tokens, const int32_t* amax,
                   int32_t* win, int32_t* pool_len, int32_t* pool, int nseq, int V, int W,
                   int N, int G, DevResult* res, hipStream_t s);
// caches [layer][nseq][Hkv][...]
void launch_kv_compact(const DevState* st, int nseq, int n_layers, int Hkv, int dh,
                       int max_ctx, int W, int N, int elem, void* k_cache,
                       void* vt_cache, hipStream_t s);
void launch_advance(DevState* st, int M, const int32_t* amax, int set_cur,
                    hipStream_t s);
// insert every N-gram of the device sequence seq[0..m), in position order
void launch_seed_pool(const int32_t* seq_dev, int m, int32_t* pool_len, int32_t* pool, int N,
                      int G, hipStream_t s);
void launch_pool_insert(DevState* st, int32_t key, const int32_t* tail_dev,
                        int32_t* pool_len, int32_t* pool, int N, int G,
                        hipStream_t s);

}  // namespace la
