// Host side of the lookahead library: configuration checks, workspace
// carve-up, weight repacking, prefill, the captured step graph and the
// inspection calls.  See include/la.h for the contract of every entry point.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "la.h"
#include "la_internal.h"

using namespace la;

namespace {

constexpr int MAX_ROWS = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Bump allocator over the caller's workspace; with base == nullptr it only
// measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

struct Layer {
  const void *anorm, *fnorm;
  const void* wqkv;  // bf16: packed tiles; f32: fused row-major copy
  const void* wo;
  const void* wgu;   // bf16: packed, gate/up tiles interleaved
  const void *wg, *wu;  // f32 originals
  const void* wd;
};

// Optional per-launch timing: HIP events recorded around each launch on the
// launch stream, summed per kernel class.
struct Prof {
  std::vector<hipEvent_t>* pool;
  std::vector<int> cat;
  size_t used = 0;
  hipStream_t s;
  void begin(int c) {
    ensure();
    cat.push_back(c);
    (void)hipEventRecord((*pool)[used++], s);
  }
  void end() {
    ensure();
    (void)hipEventRecord((*pool)[used++], s);
  }
  void ensure() {
    if (used == pool->size()) {
      hipEvent_t e;
      (void)hipEventCreate(&e);
      pool->push_back(e);
    }
  }
};

}  // namespace

struct la_ctx {
  la_config cfg;
  int T = 0, B = 1, MR = 0, bf16 = 0, elem = 4, ctx_stride = 0;
  int qdim = 0, kvdim = 0, qkv_rows = 0;
  hipStream_t stream = nullptr;
  bool poisoned = false, use_graph = true;
  std::string err;
  std::vector<int> kv_len_host;  // per sequence
  std::vector<char> prefilled;   // per sequence
  // device carve-up (per-sequence arrays: sequence 0 first)
  DevState* st = nullptr;        // [B]
  DevResult* res_dev = nullptr;  // [B]
  SampleParams* sparams = nullptr;  // [B]; zeros: argmax
  float *x = nullptr, *logits = nullptr, *rope_cos = nullptr, *rope_sin = nullptr;
  float *gpart = nullptr, *attn_po = nullptr, *attn_pml = nullptr;
  float* ssq = nullptr;  // bf16: per-row partial sums of squares (deferred RMSNorm)
  float* ssq16 = nullptr;  // bf16, passes of <= 16 rows: [16][d / 16], one per 16 columns
  float* rope_rows = nullptr;  // bf16: per block row cos[64], sin[64]
  int ssn = 1;
  void *xn = nullptr, *ffa = nullptr, *qb = nullptr;  // f32 path: row-major
  uint16_t *xnf = nullptr, *of = nullptr, *af = nullptr;  // bf16: fragment layout
  int MTT = 0;
  int32_t *tokens = nullptr, *relpos = nullptr, *amax = nullptr, *prompt_buf = nullptr;
  int32_t *win = nullptr, *pool_len = nullptr, *pool = nullptr;  // [B][...]
  size_t pool_seq = 0;        // pool ints per sequence (V * G * (N-1))
  int32_t* tail_buf = nullptr;
  void *kcache = nullptr, *vtcache = nullptr;  // [layer][B][Hkv][...]
  size_t kv_layer_elems = 0;  // elements of one layer's K (or V^T) cache, all sequences
  size_t kv_seq = 0;          // of them per sequence
  // weights
  const void *emb = nullptr, *final_norm = nullptr, *lm = nullptr;
  std::vector<Layer> layers;
  GemmPlan p_qkv{1, 1}, p_o{1, 1}, p_gu{1, 1}, p_d{1, 1}, p_lm{1, 1};
  int attn_splits = 1;
  // host
  DevResult* res_host = nullptr;  // pinned [B]: where the step's result copy lands
  // pipelined stepping: two pinned result slots, one captured step per slot
  // (the slot's copy baked into its graph), an event per slot
  DevResult* res_slot[2] = {nullptr, nullptr};
  hipGraphExec_t gexec_slot1 = nullptr;
  hipGraph_t graph_slot1 = nullptr;
  hipEvent_t slot_ev[2] = {nullptr, nullptr};
  int inflight = 0, next_slot = 0, oldest_slot = 0;
  int32_t* pin = nullptr;         // pinned staging
  size_t pin_count = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t gexec = nullptr;  // result copy into res_slot[0]
  std::vector<hipEvent_t> events;  // profiling only
};

namespace {

la_status fail(la_ctx* c, la_status s, const std::string& msg) {
  if (c) {
    c->err = msg;
    if (s == LA_ERR_HIP) c->poisoned = true;
  }
  return s;
}

#define LA_HIP(c, call)                                                          \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess)                                                        \
      return fail((c), LA_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

la_status check_config(const la_config* cfg, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return LA_ERR_INVALID_ARG; };
  auto uns = [&](const char* m) { if (why) *why = m; return LA_ERR_UNSUPPORTED; };
  if (!cfg) return bad("config is NULL");
  const la_config& c = *cfg;
  if (c.n_layers < 1 || c.d_model < 1 || c.n_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 2 ||
      c.d_ffn < 1 || c.vocab < 2 || c.max_ctx < 1)
    return bad("dimensions must be positive");
  if (c.n_heads % c.n_kv_heads) return bad("n_heads must be a multiple of n_kv_heads");
  if (c.N < 2 || c.N > 32) return bad("N must be in 2..32");
  if (c.W < 0 || c.G < 0) return bad("W and G must be >= 0");
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.f)) return bad("rms_eps and rope_theta must be > 0");
  if (c.dtype != LA_F32 && c.dtype != LA_BF16) return bad("dtype must be LA_F32 or LA_BF16");
  if (c.batch < 0) return bad("batch must be >= 0 (0 reads as 1)");
  const long B = c.batch > 0 ? c.batch : 1;
  long T = 1 + (long)(c.W + c.G) * (c.N - 1);
  if (T * B > MAX_ROWS) return uns("batch * (1 + (W+G)(N-1)) must be <= 256");
  if (c.max_ctx < T + 1) return bad("max_ctx must exceed the step's rows");
  if (c.head_dim % 2) return bad("head_dim must be even");
  if (c.dtype == LA_BF16) {
    if (c.head_dim != 128) return uns("bf16 kernels need head_dim 128");
    if (c.d_model % 128 || c.d_ffn % 64 || c.vocab % 128)
      return uns("bf16 kernels need d_model and vocab multiples of 128, d_ffn of 64");
    if (c.d_model > 8192) return uns("bf16 kernels need d_model <= 8192");
    if (c.max_ctx > (1 << 24)) return uns("bf16 kernels need max_ctx <= 16777216");
  } else {
    if (c.head_dim > 256) return uns("f32 kernels need head_dim <= 256");
    if (c.d_model % 2 || c.d_ffn % 2 || c.vocab % 2) return uns("f32 kernels need even sizes");
    if (c.max_ctx > 16384) return uns("f32 kernels need max_ctx <= 16384");
  }
  return LA_OK;
}

// Lay out (or measure) the workspace.  Returns the byte count.
size_t carve(la_ctx* c, void* base) {
  const la_config& g = c->cfg;
  Carver cv(base);
  const int d = g.d_model, V = g.vocab, F = g.d_ffn, dh = g.head_dim;
  const int B = c->B, n1 = g.N - 1;
  c->st = cv.take<DevState>(B);
  c->res_dev = cv.take<DevResult>(B);
  c->sparams = cv.take<SampleParams>(B);
  c->tail_buf = cv.take<int32_t>(32);
  c->tokens = cv.take<int32_t>(c->MR);
  c->relpos = cv.take<int32_t>(c->MR);
  c->amax = cv.take<int32_t>(c->MR);
  c->prompt_buf = cv.take<int32_t>(c->MR);
  c->win = cv.take<int32_t>((size_t)B * std::max(1, n1 * g.W));
  c->pool_len = cv.take<int32_t>((size_t)B * V);
  c->pool_seq = (size_t)V * g.G * n1;
  c->pool = cv.take<int32_t>((size_t)B * V * std::max(1, g.G) * n1);
  c->x = cv.take<float>((size_t)c->MR * d);
  c->logits = cv.take<float>((size_t)c->MR * V);
  c->rope_cos = cv.take<float>((size_t)c->ctx_stride * (dh / 2));
  c->rope_sin = cv.take<float>((size_t)c->ctx_stride * (dh / 2));
  c->kv_seq = (size_t)g.n_kv_heads * c->ctx_stride * dh;
  c->kv_layer_elems = c->kv_seq * B;
  c->kcache = cv.take<char>(c->kv_layer_elems * g.n_layers * c->elem);
  c->vtcache = cv.take<char>(c->kv_layer_elems * g.n_layers * c->elem);
  c->qb = cv.take<char>((size_t)c->MR * c->qdim * c->elem);
  if (c->bf16) {
    c->MTT = c->MR / 16;
    c->xnf = cv.take<uint16_t>((size_t)c->MR * d);
    c->of = cv.take<uint16_t>((size_t)c->MR * c->qdim);
    c->af = cv.take<uint16_t>((size_t)c->MR * F);
    const int step_rows = c->T * B;  // the plans follow the step's row count
    c->p_qkv = gemm_bf16_plan(c->qkv_rows, d, step_rows);
    c->p_o = gemm_bf16_plan(d, c->qdim, step_rows);
    c->p_gu = GemmPlan{1, (d / 32) % 2 == 0 ? 2 : 1};  // no split: SwiGLU fused
    c->p_d = gemm_bf16_plan(d, F, step_rows);
    c->p_lm = GemmPlan{1, (d / 32) % 2 == 0 ? 2 : 1};
    size_t gp = 0;
    gp = std::max(gp, (size_t)c->p_qkv.ksplit * c->MR * c->qkv_rows);
    gp = std::max(gp, (size_t)c->p_o.ksplit * c->MR * d);
    gp = std::max(gp, (size_t)c->p_d.ksplit * c->MR * d);
    c->gpart = cv.take<float>(gp);
    c->attn_splits = attn_bf16_splits(g.n_heads * B, c->T, c->ctx_stride);
    // partials [seq][H][splits][rows16]: B blocks of T rows, or one prefill chunk
    const size_t rows_all = std::max((size_t)B * ((c->T + 15) & ~15), (size_t)c->MR);
    size_t rows16 = (size_t)g.n_heads * c->attn_splits * rows_all;
    c->attn_po = cv.take<float>(rows16 * dh);
    c->attn_pml = cv.take<float>(rows16 * 2);
    c->ssq = cv.take<float>((size_t)c->MR * SSQ_STRIDE);
    c->ssq16 = cv.take<float>((size_t)16 * (d / 16));
    c->rope_rows = cv.take<float>((size_t)c->MR * 128);
    c->ssn = (d + SSQ_CHUNK - 1) / SSQ_CHUNK;
  } else {
    c->xn = cv.take<char>((size_t)c->MR * std::max(d, c->qdim) * c->elem);
    c->ffa = cv.take<char>((size_t)c->MR * F * c->elem);
  }
  // weights owned by the workspace
  c->layers.assign(g.n_layers, Layer{});
  for (int l = 0; l < g.n_layers; l++) {
    Layer& L = c->layers[l];
    L.wqkv = cv.take<char>((size_t)c->qkv_rows * d * c->elem);
    if (c->bf16) {
      L.wo = cv.take<char>((size_t)d * c->qdim * 2);
      L.wgu = cv.take<char>((size_t)2 * F * d * 2);
      L.wd = cv.take<char>((size_t)d * F * 2);
    }
  }
  if (c->bf16) c->lm = cv.take<char>((size_t)V * d * 2);
  return align_up(cv.off, 256);
}

void init_dims(la_ctx* c, const la_config* cfg) {
  c->cfg = *cfg;
  c->T = 1 + (cfg->W + cfg->G) * (cfg->N - 1);
  c->B = cfg->batch > 0 ? cfg->batch : 1;
  c->MR = std::max((int)align_up((size_t)c->T * c->B, 64), 128);
  c->bf16 = cfg->dtype == LA_BF16;
  c->elem = c->bf16 ? 2 : 4;
  c->ctx_stride = (int)align_up(cfg->max_ctx, 64);
  c->qdim = cfg->n_heads * cfg->head_dim;
  c->kvdim = cfg->n_kv_heads * cfg->head_dim;
  c->qkv_rows = c->qdim + 2 * c->kvdim;
}

// One layer's K (or V^T) cache from sequence seq on.
void* layer_k(la_ctx* c, int l, int seq = 0) {
  return (char*)c->kcache + ((size_t)l * c->kv_layer_elems + seq * c->kv_seq) * c->elem;
}
void* layer_v(la_ctx* c, int l, int seq = 0) {
  return (char*)c->vtcache + ((size_t)l * c->kv_layer_elems + seq * c->kv_seq) * c->elem;
}

// The rows of one forward pass: row t is block row t % rps of sequence
// seq0 + t / rps.  A step forwards every sequence's block (rps = T); a
// prefill chunk, rows of one sequence's prompt.
struct Pass {
  int M;       // rows
  int mode;    // MODE_STEP / MODE_CAUSAL
  int seq0, nseq, rps;
  int rows;    // rows per sequence
};
Pass step_pass(const la_ctx* c) { return Pass{c->B * c->T, MODE_STEP, 0, c->B, c->T, c->T}; }
Pass prefill_pass(const la_ctx* c, int seq, int m) { return Pass{m, MODE_CAUSAL, seq, 1, c->MR, m}; }

EpiArgs base_epi(la_ctx* c, const Pass& p) {
  EpiArgs ea;
  memset(&ea, 0, sizeof(ea));
  ea.M = p.M;
  ea.st = c->st + p.seq0;
  ea.rps = p.rps;
  ea.kv_seq = c->kv_seq;
  ea.relpos = c->relpos;
  ea.rope_cos = c->rope_cos;
  ea.rope_sin = c->rope_sin;
  ea.qdim = c->qdim;
  ea.kvdim = c->kvdim;
  ea.dh = c->cfg.head_dim;
  ea.max_ctx = c->ctx_stride;
  return ea;
}

AttnArgs attn_args(la_ctx* c, int l, const Pass& p) {
  const la_config& g = c->cfg;
  AttnArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.q = c->qb;
  aa.k_cache = layer_k(c, l, p.seq0);
  aa.vt_cache = layer_v(c, l, p.seq0);
  aa.out = c->bf16 ? (void*)c->of : c->xn;
  aa.out_mtt = c->bf16 ? c->MTT : 0;
  aa.st = c->st + p.seq0;
  aa.M = p.rows;
  aa.rps = p.rps;
  aa.nseq = p.nseq;
  aa.kv_seq = c->kv_seq;
  aa.mode = p.mode;
  aa.H = g.n_heads;
  aa.Hkv = g.n_kv_heads;
  aa.dh = g.head_dim;
  aa.ctx_stride = c->ctx_stride;
  aa.W = g.W;
  aa.N = g.N;
  aa.part_o = c->attn_po;
  aa.part_ml = c->attn_pml;
  aa.splits = c->attn_splits;
  // the caches are zero-filled at creation and the steps write only
  // projections into them: every V^T entry, also past the context, is finite
  aa.vt_finite = 1;
  return aa;
}

// Passes of at most SMALL_PASS_ROWS rows of models up to SMALL_PASS_DMODEL
// wide take the one-tile GEMMs, whose epilogues replace the K-split reduce
// kernels.  Their activation loads grow with the rows (M x 64 bytes beside
// each 1 KiB weight tile), so the gain shrinks as the rows grow.  Measured
// (same-process A/Bs, ms per step, K-split path / one-tile path): 7B shape,
// plain batched decode, 1 row 3.28 / 2.91, 4 rows 3.44 / 3.08, 8 rows 3.49
// / 3.30, 12 rows 3.55 / 3.48, 16 rows 3.63 / 3.71.  On wider models the
// K-split GEMMs fill the CUs (7B leaves a third of them idle in QKV and
// gate/up) and stream faster than the one-tile kernel, more than the reduce
// kernels cost: plain decode 13B shape 5.51 / 5.85, 34B shape 12.0 / 12.6.
constexpr int SMALL_PASS_ROWS = 12;
constexpr int SMALL_PASS_DMODEL = 4096;
bool small_pass(const la_ctx* c, int M) {
  const la_config& g = c->cfg;
  const int d = g.d_model, F = g.d_ffn;
  return M <= SMALL_PASS_ROWS && d <= SMALL_PASS_DMODEL && gemv_bf16_ok(M, c->qkv_rows, d) &&
         gemv_bf16_ok(M, d, c->qdim) &&
         gemv_bf16_ok(M, 2 * F, d) && gemv_bf16_ok(M, d, F);
}

// One launch of layer l's kernel class k (QKV, ATTN, O, GATEUP or DOWN) in
// a pass of at most 16 rows.  The first layer's QKV reads the sums of
// squares the assembly wrote (per SSQ_CHUNK columns); every later norm
// input was written by an O or down epilogue (per 16 columns, ssq16).
void launch_small(la_ctx* c, const Pass& p, int l, int k, const EpiArgs& ea, hipStream_t s) {
  const la_config& g = c->cfg;
  const int d = g.d_model, F = g.d_ffn;
  const Layer& L = c->layers[l];
  GemvArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.MTT = c->MTT;
  ga.M = p.M;
  ga.eps = g.rms_eps;
  ga.d_in = d;
  switch (k) {
    case LA_PROF_QKV:
      ga.X = c->xnf;
      ga.Wp = (const uint16_t*)L.wqkv;
      ga.K = d;
      ga.N = c->qkv_rows;
      ga.ssq = l == 0 ? c->ssq : c->ssq16;
      ga.ssq_n = l == 0 ? c->ssn : d / 16;
      ga.ssq_stride = l == 0 ? SSQ_STRIDE : d / 16;
      ga.ea = ea;
      launch_gemv_bf16(EPI_QKV, ga, s);
      break;
    case LA_PROF_ATTN:
      launch_attn_bf16(attn_args(c, l, p), s);
      break;
    case LA_PROF_O:
      ga.X = c->of;
      ga.Wp = (const uint16_t*)L.wo;
      ga.K = c->qdim;
      ga.N = d;
      ga.x = c->x;
      ga.wn = (const uint16_t*)L.fnorm;
      ga.xnf = c->xnf;
      ga.ssq_out = c->ssq16;
      launch_gemv_bf16(EPI_RESID, ga, s);
      break;
    case LA_PROF_GATEUP:
      ga.X = c->xnf;
      ga.Wp = (const uint16_t*)L.wgu;
      ga.K = d;
      ga.N = 2 * F;
      ga.ssq = c->ssq16;
      ga.ssq_n = d / 16;
      ga.ssq_stride = d / 16;
      ga.act = c->af;
      launch_gemv_bf16(EPI_SWIGLU, ga, s);
      break;
    default: {  // down; the last layer's next norm is the final one, applied whole afterwards
      const bool last = l + 1 == g.n_layers;
      ga.X = c->af;
      ga.Wp = (const uint16_t*)L.wd;
      ga.K = F;
      ga.N = d;
      ga.x = c->x;
      ga.wn = last ? nullptr : (const uint16_t*)c->layers[l + 1].anorm;
      ga.xnf = last ? nullptr : c->xnf;
      ga.ssq_out = c->ssq16;
      launch_gemv_bf16(EPI_RESID, ga, s);
      break;
    }
  }
}

// The decoder over the assembled rows.  bf16: x holds their embeddings and
// xnf the first layer's normalized input; f32: x only.
void enqueue_layers(la_ctx* c, const Pass& p, hipStream_t s, Prof* pf = nullptr) {
#define P_BEGIN(k) if (pf) pf->begin(k)
#define P_END() if (pf) pf->end()
  const la_config& g = c->cfg;
  const int d = g.d_model, F = g.d_ffn, M = p.M;
  for (int l = 0; l < g.n_layers; l++) {
    const Layer& L = c->layers[l];
    EpiArgs ea = base_epi(c, p);
    ea.out_act = c->qb;
    ea.k_cache = layer_k(c, l, p.seq0);
    ea.vt_cache = layer_v(c, l, p.seq0);
    ea.ssq = c->ssq;
    ea.rope_rows = c->rope_rows;
    ea.ssn = c->ssn;
    ea.dmodel = d;
    ea.eps = g.rms_eps;
    if (c->bf16 && small_pass(c, M)) {
      const uint16_t* next_norm =
          (const uint16_t*)(l + 1 < g.n_layers ? c->layers[l + 1].anorm : c->final_norm);
      for (int k = LA_PROF_QKV; k <= LA_PROF_DOWN; k++) {
        P_BEGIN(k);
        launch_small(c, p, l, k, ea, s);
        P_END();
      }
      if (l + 1 == g.n_layers) {  // the LM head takes fully normalized rows
        P_BEGIN(LA_PROF_REDUCE);
        launch_red_resid_norm(nullptr, 0, d, M, c->x, next_norm, g.rms_eps, c->xnf, c->MTT, s);
        P_END();
      }
    } else if (c->bf16) {
      const uint16_t* next_norm =
          (const uint16_t*)(l + 1 < g.n_layers ? c->layers[l + 1].anorm : c->final_norm);
      P_BEGIN(LA_PROF_QKV);
      launch_gemm_bf16(c->xnf, c->MTT, (const uint16_t*)L.wqkv, d, c->qkv_rows, M, c->p_qkv,
                       c->gpart, s);
      P_END();
      P_BEGIN(LA_PROF_REDUCE);
      launch_red_qkv(c->gpart, c->p_qkv.ksplit, c->qkv_rows, M, ea, s);
      P_END();
      P_BEGIN(LA_PROF_ATTN);
      launch_attn_bf16(attn_args(c, l, p), s);
      P_END();
      P_BEGIN(LA_PROF_O);
      launch_gemm_bf16(c->of, c->MTT, (const uint16_t*)L.wo, c->qdim, d, M, c->p_o, c->gpart, s);
      P_END();
      P_BEGIN(LA_PROF_REDUCE);
      launch_red_resid_scale(c->gpart, c->p_o.ksplit, d, M, c->x, (const uint16_t*)L.fnorm,
                             c->xnf, c->MTT, c->ssq, s);
      P_END();
      P_BEGIN(LA_PROF_GATEUP);
      launch_gemm_bf16_swiglu(c->xnf, c->MTT, (const uint16_t*)L.wgu, d, 2 * F, M, c->p_gu.J,
                              c->af, c->ssq, c->ssn, g.rms_eps, s);
      P_END();
      P_BEGIN(LA_PROF_DOWN);
      launch_gemm_bf16(c->af, c->MTT, (const uint16_t*)L.wd, F, d, M, c->p_d, c->gpart, s);
      P_END();
      P_BEGIN(LA_PROF_REDUCE);
      if (l + 1 < g.n_layers)  // the next layer's QKV reduce applies the row scale
        launch_red_resid_scale(c->gpart, c->p_d.ksplit, d, M, c->x, next_norm, c->xnf, c->MTT,
                               c->ssq, s);
      else  // the LM head takes fully normalized rows
        launch_red_resid_norm(c->gpart, c->p_d.ksplit, d, M, c->x, next_norm, g.rms_eps,
                              c->xnf, c->MTT, s);
      P_END();
    } else {
      P_BEGIN(LA_PROF_REDUCE);
      launch_rmsnorm(c->x, L.anorm, M, d, g.rms_eps, 0, c->xn, s);
      P_END();
      P_BEGIN(LA_PROF_QKV);
      launch_gemm_f32(EPI_QKV, (const float*)c->xn, (const float*)L.wqkv, nullptr, d,
                      c->qkv_rows, M, ea, s);
      P_END();
      P_BEGIN(LA_PROF_ATTN);
      launch_attn_f32(attn_args(c, l, p), s);
      P_END();
      ea = base_epi(c, p);
      ea.out_f32 = c->x;
      ea.ld_out = d;
      P_BEGIN(LA_PROF_O);
      launch_gemm_f32(EPI_RESID, (const float*)c->xn, (const float*)L.wo, nullptr, c->qdim, d, M,
                      ea, s);
      P_END();
      P_BEGIN(LA_PROF_REDUCE);
      launch_rmsnorm(c->x, L.fnorm, M, d, g.rms_eps, 0, c->xn, s);
      P_END();
      ea = base_epi(c, p);
      ea.out_act = c->ffa;
      ea.ld_out = F;
      P_BEGIN(LA_PROF_GATEUP);
      launch_gemm_f32(EPI_SWIGLU, (const float*)c->xn, (const float*)L.wg, (const float*)L.wu, d,
                      F, M, ea, s);
      P_END();
      ea = base_epi(c, p);
      ea.out_f32 = c->x;
      ea.ld_out = d;
      P_BEGIN(LA_PROF_DOWN);
      launch_gemm_f32(EPI_RESID, (const float*)c->ffa, (const float*)L.wd, nullptr, F, d, M, ea,
                      s);
      P_END();
    }
  }
}

void enqueue_head(la_ctx* c, const Pass& p, hipStream_t s, Prof* pf = nullptr) {
  const la_config& g = c->cfg;
  const int M = p.M;
  if (c->bf16 && small_pass(c, M) && g.vocab % 16 == 0) {
    // xnf already holds the final-norm'd rows
    GemvArgs ga;
    memset(&ga, 0, sizeof(ga));
    ga.X = c->xnf;
    ga.MTT = c->MTT;
    ga.Wp = (const uint16_t*)c->lm;
    ga.K = g.d_model;
    ga.N = g.vocab;
    ga.M = M;
    ga.logits = c->logits;
    P_BEGIN(LA_PROF_LMHEAD);
    launch_gemv_bf16(EPI_LOGITS, ga, s);
    P_END();
  } else if (c->bf16) {
    // xnf already holds the final-norm'd rows
    P_BEGIN(LA_PROF_LMHEAD);
    launch_gemm_bf16(c->xnf, c->MTT, (const uint16_t*)c->lm, g.d_model, g.vocab, M, c->p_lm,
                     c->logits, s);
    P_END();
  } else {
    P_BEGIN(LA_PROF_REDUCE);
    launch_rmsnorm(c->x, c->final_norm, M, g.d_model, g.rms_eps, 0, c->xn, s);
    P_END();
    EpiArgs ea = base_epi(c, Pass{M, MODE_STEP, 0, 1, M, M});
    ea.out_f32 = c->logits;
    ea.ld_out = g.vocab;
    P_BEGIN(LA_PROF_LMHEAD);
    launch_gemm_f32(EPI_LOGITS, (const float*)c->xn, (const float*)c->lm, nullptr, g.d_model,
                    g.vocab, M, ea, s);
    P_END();
  }
  // each row's token: the argmax, or the draw the sequence's sampling asks for
  P_BEGIN(LA_PROF_OTHER);
  launch_select(c->logits, M, g.vocab, c->T, p.mode, g.W, g.N, c->st + p.seq0, c->relpos,
                c->sparams + p.seq0, c->amax, s);
  P_END();
}

void enqueue_step(la_ctx* c, hipStream_t s, Prof* pf = nullptr) {
  const la_config& g = c->cfg;
  const Pass p = step_pass(c);
  P_BEGIN(LA_PROF_OTHER);
  launch_assemble(MODE_STEP, c->st, c->win, c->pool_len, c->pool, nullptr, p.M, c->T, g.vocab,
                  g.W, g.N, g.G, c->tokens, c->relpos, c->st, c->emb, g.d_model, c->bf16, c->x,
                  (const uint16_t*)c->layers[0].anorm, g.rms_eps, c->xnf, c->MTT, c->ssq,
                  c->rope_cos, c->rope_sin, c->rope_rows, s);
  P_END();
  enqueue_layers(c, p, s, pf);
  enqueue_head(c, p, s, pf);
  P_BEGIN(LA_PROF_OTHER);
  launch_verify(c->st, c->tokens, c->amax, c->win, c->pool_len, c->pool, c->B, g.vocab, g.W,
                g.N, g.G, c->res_dev, s);
  P_END();
  P_BEGIN(LA_PROF_OTHER);
  launch_kv_compact(c->st, c->B, g.n_layers, g.n_kv_heads, g.head_dim, c->ctx_stride, g.W, g.N,
                    c->elem, c->kcache, c->vtcache, s);
  P_END();
  (void)hipMemcpyAsync(c->res_host, c->res_dev, sizeof(DevResult) * c->B, hipMemcpyDeviceToHost,
                       s);
}
#undef P_BEGIN
#undef P_END

la_status check_alive(la_ctx* c) {
  if (!c) return LA_ERR_INVALID_ARG;
  if (c->poisoned) return fail(c, LA_ERR_STATE, "context poisoned by an earlier HIP failure: " + c->err);
  return LA_OK;
}

// Usable for every call but the pipelined pair: alive, no step in flight.
la_status check_usable(la_ctx* c) {
  const la_status us = check_alive(c);
  if (us != LA_OK) return us;
  if (c->inflight) return fail(c, LA_ERR_STATE, "steps submitted and not collected");
  return LA_OK;
}

// Every sequence prefilled and room for one more step in each.
la_status check_steppable(la_ctx* c, const char* what) {
  for (int b = 0; b < c->B; b++)
    if (!c->prefilled[b])
      return fail(c, LA_ERR_STATE, std::string(what) + " before every sequence was prefilled");
  for (int b = 0; b < c->B; b++)
    if ((long)c->kv_len_host[b] + c->T > c->cfg.max_ctx)
      return fail(c, LA_ERR_OUT_OF_CAPACITY, "kv_len + step rows exceed max_ctx");
  return LA_OK;
}

void take_results(la_ctx* c, la_step_result* out) {
  static_assert(sizeof(DevResult) == sizeof(la_step_result), "result layout");
  memcpy(out, c->res_host, sizeof(*out) * c->B);
  for (int b = 0; b < c->B; b++) c->kv_len_host[b] = out[b].kv_len;
}

}  // namespace

extern "C" {

const char* la_status_string(la_status s) {
  switch (s) {
    case LA_OK: return "ok";
    case LA_ERR_INVALID_ARG: return "invalid argument";
    case LA_ERR_STATE: return "invalid state";
    case LA_ERR_OUT_OF_CAPACITY: return "out of capacity";
    case LA_ERR_HIP: return "HIP error";
    case LA_ERR_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* la_last_error(const la_ctx* c) { return c ? c->err.c_str() : "no context"; }

int32_t la_step_rows(const la_ctx* c) { return c ? c->T : 0; }

size_t la_workspace_bytes(const la_config* cfg) {
  if (check_config(cfg, nullptr) != LA_OK) return 0;
  la_ctx tmp;
  init_dims(&tmp, cfg);
  return carve(&tmp, nullptr);
}

la_status la_create(const la_config* cfg, const void* const* weights, void* workspace,
                    size_t workspace_bytes, void* hip_stream, la_ctx** out) {
  if (!out) return LA_ERR_INVALID_ARG;
  *out = nullptr;
  std::string why;
  la_status vs = check_config(cfg, &why);
  if (vs != LA_OK) return vs;
  if (!weights || !workspace) return LA_ERR_INVALID_ARG;
  const int nw = 3 + 9 * cfg->n_layers;
  for (int i = 0; i < nw; i++)
    if (!weights[i]) return LA_ERR_INVALID_ARG;
  la_ctx* c = new la_ctx();
  init_dims(c, cfg);
  size_t need = carve(c, nullptr);
  if (workspace_bytes < need) {
    delete c;
    return LA_ERR_OUT_OF_CAPACITY;
  }
  carve(c, workspace);
  c->stream = (hipStream_t)hip_stream;
  const char* ng = getenv("LA_NO_GRAPH");
  c->use_graph = !(ng && ng[0] == '1');
  *out = c;
  hipStream_t s = c->stream;
  const la_config& g = c->cfg;
  const int d = g.d_model, F = g.d_ffn, V = g.vocab, dh = g.head_dim;

  // pinned host buffers
  c->pin_count = std::max<size_t>(c->MR, (size_t)std::max(1, (g.N - 1) * g.W)) + 64;
  LA_HIP(c, hipHostMalloc((void**)&c->res_host, sizeof(DevResult) * c->B, hipHostMallocDefault));
  LA_HIP(c, hipHostMalloc((void**)&c->res_slot[1], sizeof(DevResult) * c->B, hipHostMallocDefault));
  c->res_slot[0] = c->res_host;
  memset(c->res_slot[1], 0, sizeof(DevResult) * c->B);
  for (int i = 0; i < 2; i++) LA_HIP(c, hipEventCreateWithFlags(&c->slot_ev[i], hipEventDisableTiming));
  LA_HIP(c, hipHostMalloc((void**)&c->pin, c->pin_count * sizeof(int32_t), hipHostMallocDefault));
  memset(c->res_host, 0, sizeof(DevResult) * c->B);
  c->kv_len_host.assign(c->B, 0);
  c->prefilled.assign(c->B, 0);

  // clear state, caches and activations (fill kernels: finite padding rows)
  launch_fill_u32(workspace, 0, need / 4, s);

  // rotary tables: angle = pos * theta^(-2i/dh), computed in double
  {
    std::vector<float> cs((size_t)c->ctx_stride * (dh / 2)), sn(cs.size());
    for (int p = 0; p < c->ctx_stride; p++)
      for (int i = 0; i < dh / 2; i++) {
        double ang = (double)p * pow((double)g.rope_theta, -2.0 * i / dh);
        cs[(size_t)p * (dh / 2) + i] = (float)cos(ang);
        sn[(size_t)p * (dh / 2) + i] = (float)sin(ang);
      }
    LA_HIP(c, hipMemcpyAsync(c->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, s));
    LA_HIP(c, hipMemcpyAsync(c->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, s));
    LA_HIP(c, hipStreamSynchronize(s));
  }

  // weights
  c->emb = weights[0];
  c->final_norm = weights[1];
  for (int l = 0; l < g.n_layers; l++) {
    const void* const* lw = weights + 3 + 9 * l;
    Layer& L = c->layers[l];
    L.anorm = lw[0];
    L.fnorm = lw[5];
    L.wg = lw[6];
    L.wu = lw[7];
    if (c->bf16) {
      uint16_t* q = (uint16_t*)L.wqkv;
      launch_repack_bf16((const uint16_t*)lw[1], c->qdim, d, q, 0, 1, s);
      launch_repack_bf16((const uint16_t*)lw[2], c->kvdim, d, q, c->qdim / 16, 1, s);
      launch_repack_bf16((const uint16_t*)lw[3], c->kvdim, d, q, (c->qdim + c->kvdim) / 16, 1, s);
      launch_repack_bf16((const uint16_t*)lw[4], d, c->qdim, (uint16_t*)L.wo, 0, 1, s);
      launch_repack_bf16((const uint16_t*)lw[6], F, d, (uint16_t*)L.wgu, 0, 2, s);
      launch_repack_bf16((const uint16_t*)lw[7], F, d, (uint16_t*)L.wgu, 1, 2, s);
      launch_repack_bf16((const uint16_t*)lw[8], d, F, (uint16_t*)L.wd, 0, 1, s);
    } else {
      char* q = (char*)L.wqkv;
      LA_HIP(c, hipMemcpyAsync(q, lw[1], (size_t)c->qdim * d * 4, hipMemcpyDeviceToDevice, s));
      LA_HIP(c, hipMemcpyAsync(q + (size_t)c->qdim * d * 4, lw[2], (size_t)c->kvdim * d * 4,
                               hipMemcpyDeviceToDevice, s));
      LA_HIP(c, hipMemcpyAsync(q + (size_t)(c->qdim + c->kvdim) * d * 4, lw[3],
                               (size_t)c->kvdim * d * 4, hipMemcpyDeviceToDevice, s));
      L.wo = lw[4];
      L.wd = lw[8];
    }
  }
  if (c->bf16) launch_repack_bf16((const uint16_t*)weights[2], V, d, (uint16_t*)c->lm, 0, 1, s);
  else c->lm = weights[2];
  LA_HIP(c, hipGetLastError());
  LA_HIP(c, hipStreamSynchronize(s));

  // capture the step
  if (c->use_graph) {
    hipStream_t cs;
    LA_HIP(c, hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
      enqueue_step(c, cs);
      e = hipStreamEndCapture(cs, &c->graph);
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&c->gexec, c->graph, nullptr, nullptr, 0);
    // the same step with its result copy into slot 1 (pipelined stepping)
    if (e == hipSuccess) {
      c->res_host = c->res_slot[1];
      e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
      if (e == hipSuccess) {
        enqueue_step(c, cs);
        e = hipStreamEndCapture(cs, &c->graph_slot1);
      }
      c->res_host = c->res_slot[0];
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&c->gexec_slot1, c->graph_slot1, nullptr, nullptr, 0);
    (void)hipStreamDestroy(cs);
    if (e != hipSuccess) return fail(c, LA_ERR_HIP, std::string("step graph capture: ") + hipGetErrorString(e));
  }
  return LA_OK;
}

la_status la_prefill(la_ctx* c, const int32_t* prompt, int32_t n_prompt, const int32_t* init_window,
                     int32_t* first_token) {
  return la_prefill_seq(c, 0, prompt, n_prompt, init_window, first_token);
}

la_status la_prefill_seq(la_ctx* c, int32_t seq, const int32_t* prompt, int32_t n_prompt,
                         const int32_t* init_window, int32_t* first_token) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  const la_config& g = c->cfg;
  if (seq < 0 || seq >= c->B) return fail(c, LA_ERR_INVALID_ARG, "seq out of range");
  if (!prompt || n_prompt < 1 || !first_token) return fail(c, LA_ERR_INVALID_ARG, "prompt/first_token");
  if (g.W > 0 && !init_window) return fail(c, LA_ERR_INVALID_ARG, "init_window required when W > 0");
  for (int i = 0; i < n_prompt; i++)
    if (prompt[i] < 0 || prompt[i] >= g.vocab) return fail(c, LA_ERR_INVALID_ARG, "prompt token out of range");
  const int nwin = (g.N - 1) * g.W;
  for (int i = 0; i < nwin; i++)
    if (init_window[i] < 0 || init_window[i] >= g.vocab) return fail(c, LA_ERR_INVALID_ARG, "window token out of range");
  if ((long)n_prompt + c->T > g.max_ctx) return fail(c, LA_ERR_OUT_OF_CAPACITY, "prompt + step rows exceed max_ctx");
  hipStream_t s = c->stream;
  DevState* sst = c->st + seq;
  c->prefilled[seq] = 0;
  launch_fill_u32(sst, 0, sizeof(DevState) / 4, s);
  launch_fill_u32(c->pool_len + (size_t)seq * g.vocab, 0, (size_t)g.vocab, s);
  if (nwin > 0) {
    memcpy(c->pin, init_window, sizeof(int32_t) * nwin);
    LA_HIP(c, hipMemcpyAsync(c->win + (size_t)seq * nwin, c->pin, sizeof(int32_t) * nwin,
                             hipMemcpyHostToDevice, s));
    LA_HIP(c, hipStreamSynchronize(s));
  }
  for (int p0 = 0; p0 < n_prompt; p0 += c->MR) {
    const int m = std::min(c->MR, n_prompt - p0);
    const bool last = p0 + m == n_prompt;
    memcpy(c->pin, prompt + p0, sizeof(int32_t) * m);
    LA_HIP(c, hipMemcpyAsync(c->prompt_buf, c->pin, sizeof(int32_t) * m, hipMemcpyHostToDevice, s));
    launch_assemble(MODE_CAUSAL, sst, nullptr, nullptr, nullptr, c->prompt_buf, m, m, g.vocab,
                    g.W, g.N, g.G, c->tokens, c->relpos, sst, c->emb, g.d_model, c->bf16, c->x,
                    (const uint16_t*)c->layers[0].anorm, g.rms_eps, c->xnf, c->MTT, c->ssq,
                    c->rope_cos, c->rope_sin, c->rope_rows, s);
    const Pass pp = prefill_pass(c, seq, m);
    enqueue_layers(c, pp, s);
    if (last) enqueue_head(c, pp, s);
    launch_advance(sst, m, c->amax, last ? 1 : 0, s);
    LA_HIP(c, hipGetLastError());
    LA_HIP(c, hipStreamSynchronize(s));
  }
  DevState hs;
  LA_HIP(c, hipMemcpy(&hs, sst, sizeof(hs), hipMemcpyDeviceToHost));
  c->kv_len_host[seq] = hs.L;
  *first_token = hs.cur;
  c->prefilled[seq] = 1;
  return LA_OK;
}


la_status la_step(la_ctx* c, la_step_result* out) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  if (!out) return fail(c, LA_ERR_INVALID_ARG, "out is NULL");
  us = check_steppable(c, "la_step");
  if (us != LA_OK) return us;
  if (c->use_graph) {
    LA_HIP(c, hipGraphLaunch(c->gexec, c->stream));
  } else {
    enqueue_step(c, c->stream);
    LA_HIP(c, hipGetLastError());
  }
  LA_HIP(c, hipStreamSynchronize(c->stream));
  take_results(c, out);
  return LA_OK;
}

la_status la_step_submit(la_ctx* c) {
  la_status us = check_alive(c);
  if (us != LA_OK) return us;
  if (c->inflight == 2) return fail(c, LA_ERR_STATE, "two steps in flight: collect one first");
  for (int b = 0; b < c->B; b++)
    if (!c->prefilled[b]) return fail(c, LA_ERR_STATE, "la_step_submit before every sequence was prefilled");
  // a step commits at most N tokens; steps in flight have not reported theirs
  for (int b = 0; b < c->B; b++)
    if ((long)c->kv_len_host[b] + (long)c->inflight * c->cfg.N + c->T > c->cfg.max_ctx)
      return fail(c, LA_ERR_OUT_OF_CAPACITY, "kv_len + steps in flight + step rows exceed max_ctx");
  const int slot = c->next_slot;
  if (c->use_graph) {
    LA_HIP(c, hipGraphLaunch(slot ? c->gexec_slot1 : c->gexec, c->stream));
  } else {
    c->res_host = c->res_slot[slot];
    enqueue_step(c, c->stream);
    c->res_host = c->res_slot[0];
    LA_HIP(c, hipGetLastError());
  }
  LA_HIP(c, hipEventRecord(c->slot_ev[slot], c->stream));
  c->next_slot ^= 1;
  c->inflight++;
  return LA_OK;
}

la_status la_step_collect(la_ctx* c, la_step_result* out) {
  la_status us = check_alive(c);
  if (us != LA_OK) return us;
  if (!out) return fail(c, LA_ERR_INVALID_ARG, "out is NULL");
  if (!c->inflight) return fail(c, LA_ERR_STATE, "no step in flight");
  const int slot = c->oldest_slot;
  LA_HIP(c, hipEventSynchronize(c->slot_ev[slot]));
  memcpy(out, c->res_slot[slot], sizeof(*out) * c->B);
  for (int b = 0; b < c->B; b++) c->kv_len_host[b] = out[b].kv_len;
  c->oldest_slot ^= 1;
  c->inflight--;
  return LA_OK;
}

la_status la_profile_step(la_ctx* c, float* ms, int32_t* launches, la_step_result* out) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  if (!out || !ms || !launches) return fail(c, LA_ERR_INVALID_ARG, "NULL output");
  us = check_steppable(c, "la_profile_step");
  if (us != LA_OK) return us;
  LA_HIP(c, hipStreamSynchronize(c->stream));
  Prof pf;
  pf.pool = &c->events;
  pf.s = c->stream;
  enqueue_step(c, c->stream, &pf);
  LA_HIP(c, hipGetLastError());
  LA_HIP(c, hipStreamSynchronize(c->stream));
  for (int k = 0; k < LA_PROF_CLASSES; k++) {
    ms[k] = 0.f;
    launches[k] = 0;
  }
  for (size_t i = 0; i < pf.cat.size(); i++) {
    float t = 0.f;
    LA_HIP(c, hipEventElapsedTime(&t, c->events[2 * i], c->events[2 * i + 1]));
    ms[pf.cat[i]] += t;
    launches[pf.cat[i]] += 1;
  }
  take_results(c, out);
  return LA_OK;
}

la_status la_profile_kernel(la_ctx* c, int32_t klass, int32_t reps, float* us_per_launch) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  if (!us_per_launch || reps < 1 || reps > 100000)
    return fail(c, LA_ERR_INVALID_ARG, "reps must be in 1..100000 and the output non-NULL");
  for (int b = 0; b < c->B; b++)
    if (!c->prefilled[b]) return fail(c, LA_ERR_STATE, "la_profile_kernel before la_prefill");
  if (!c->bf16) return fail(c, LA_ERR_UNSUPPORTED, "la_profile_kernel needs the bf16 kernels");
  if (klass != LA_PROF_QKV && klass != LA_PROF_ATTN && klass != LA_PROF_O &&
      klass != LA_PROF_GATEUP && klass != LA_PROF_DOWN)
    return fail(c, LA_ERR_INVALID_ARG, "klass must be QKV, ATTN, O, GATEUP or DOWN");
  const la_config& g = c->cfg;
  const Pass p = step_pass(c);
  const int d = g.d_model, F = g.d_ffn, M = p.M;
  const hipStream_t s = c->stream;
  // launch i runs layer i % n_layers, so the weights streamed differ from
  // one launch to the next (no help from the last-level cache)
  const bool small = small_pass(c, M);
  auto launch = [&](int l) {
    const Layer& L = c->layers[l];
    if (small) {
      EpiArgs ea = base_epi(c, p);
      ea.out_act = c->qb;
      ea.k_cache = layer_k(c, l, p.seq0);
      ea.vt_cache = layer_v(c, l, p.seq0);
      ea.rope_rows = c->rope_rows;
      launch_small(c, p, l, klass, ea, s);
      return;
    }
    switch (klass) {
      case LA_PROF_QKV:
        launch_gemm_bf16(c->xnf, c->MTT, (const uint16_t*)L.wqkv, d, c->qkv_rows, M, c->p_qkv,
                         c->gpart, s);
        break;
      case LA_PROF_ATTN:
        launch_attn_bf16(attn_args(c, l, p), s);
        break;
      case LA_PROF_O:
        launch_gemm_bf16(c->of, c->MTT, (const uint16_t*)L.wo, c->qdim, d, M, c->p_o, c->gpart, s);
        break;
      case LA_PROF_GATEUP:
        launch_gemm_bf16_swiglu(c->xnf, c->MTT, (const uint16_t*)L.wgu, d, 2 * F, M, c->p_gu.J,
                                c->af, c->ssq, c->ssn, g.rms_eps, s);
        break;
      default:
        launch_gemm_bf16(c->af, c->MTT, (const uint16_t*)L.wd, F, d, M, c->p_d, c->gpart, s);
        break;
    }
  };
  while (c->events.size() < 2) {
    hipEvent_t e;
    LA_HIP(c, hipEventCreate(&e));
    c->events.push_back(e);
  }
  LA_HIP(c, hipStreamSynchronize(s));
  LA_HIP(c, hipEventRecord(c->events[0], s));
  for (int i = 0; i < reps; i++) launch(i % g.n_layers);
  LA_HIP(c, hipEventRecord(c->events[1], s));
  LA_HIP(c, hipGetLastError());
  LA_HIP(c, hipEventSynchronize(c->events[1]));
  float ms = 0.f;
  LA_HIP(c, hipEventElapsedTime(&ms, c->events[0], c->events[1]));
  *us_per_launch = ms * 1e3f / reps;
  return LA_OK;
}

la_status la_set_sampling(la_ctx* c, int32_t seq, float temperature, int32_t top_k, float top_p,
                          uint64_t seed) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  if (seq < 0 || seq >= c->B) return fail(c, LA_ERR_INVALID_ARG, "seq out of range");
  if (!(temperature >= 0.f) || !std::isfinite(temperature) || top_k < 0 ||
      !(top_p > 0.f && top_p <= 1.f))
    return fail(c, LA_ERR_INVALID_ARG, "temperature >= 0, top_k >= 0, 0 < top_p <= 1");
  if (temperature > 0.f && c->cfg.vocab > SAMPLE_MAX_VOCAB)
    return fail(c, LA_ERR_UNSUPPORTED, "sampling needs vocab <= 32768");
  SampleParams h;
  memset(&h, 0, sizeof(h));
  h.temperature = temperature;
  h.top_k = top_k;
  h.top_p = top_p;
  h.seed_lo = (uint32_t)seed;
  h.seed_hi = (uint32_t)(seed >> 32);
  LA_HIP(c, hipStreamSynchronize(c->stream));
  LA_HIP(c, hipMemcpy(c->sparams + seq, &h, sizeof(h), hipMemcpyHostToDevice));
  return LA_OK;
}

la_status la_destroy(la_ctx* c) {
  if (!c) return LA_OK;
  (void)hipStreamSynchronize(c->stream);
  if (c->gexec) (void)hipGraphExecDestroy(c->gexec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  if (c->gexec_slot1) (void)hipGraphExecDestroy(c->gexec_slot1);
  if (c->graph_slot1) (void)hipGraphDestroy(c->graph_slot1);
  for (hipEvent_t e : c->slot_ev)
    if (e) (void)hipEventDestroy(e);
  if (c->res_slot[1]) (void)hipHostFree(c->res_slot[1]);
  for (hipEvent_t e : c->events) (void)hipEventDestroy(e);
  if (c->res_host) (void)hipHostFree(c->res_host);
  if (c->pin) (void)hipHostFree(c->pin);
  delete c;
  return LA_OK;
}

la_status la_debug_logits(la_ctx* c, float* host, size_t n) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  size_t need = (size_t)c->B * c->T * c->cfg.vocab;
  if (!host || n < need) return fail(c, LA_ERR_INVALID_ARG, "logits buffer too small");
  LA_HIP(c, hipStreamSynchronize(c->stream));
  LA_HIP(c, hipMemcpy(host, c->logits, need * sizeof(float), hipMemcpyDeviceToHost));
  return LA_OK;
}

la_status la_debug_block(la_ctx* c, int32_t* tokens, int32_t* amax) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  LA_HIP(c, hipStreamSynchronize(c->stream));
  const size_t rows = (size_t)c->B * c->T;
  if (tokens) LA_HIP(c, hipMemcpy(tokens, c->tokens, sizeof(int32_t) * rows, hipMemcpyDeviceToHost));
  if (amax) LA_HIP(c, hipMemcpy(amax, c->amax, sizeof(int32_t) * rows, hipMemcpyDeviceToHost));
  return LA_OK;
}

la_status la_debug_window(la_ctx* c, int32_t* win) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  const int n = (c->cfg.N - 1) * c->cfg.W;
  if (n == 0) return LA_OK;
  if (!win) return fail(c, LA_ERR_INVALID_ARG, "win is NULL");
  LA_HIP(c, hipStreamSynchronize(c->stream));
  LA_HIP(c, hipMemcpy(win, c->win, sizeof(int32_t) * n * c->B, hipMemcpyDeviceToHost));
  return LA_OK;
}

la_status la_debug_pool(la_ctx* c, int32_t* len, int32_t* tails) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  const la_config& g = c->cfg;
  LA_HIP(c, hipStreamSynchronize(c->stream));
  if (len)
    LA_HIP(c, hipMemcpy(len, c->pool_len, sizeof(int32_t) * g.vocab * c->B, hipMemcpyDeviceToHost));
  if (tails && g.G > 0)
    LA_HIP(c, hipMemcpy(tails, c->pool, sizeof(int32_t) * c->pool_seq * c->B, hipMemcpyDeviceToHost));
  return LA_OK;
}

la_status la_seed_pool(la_ctx* c, const int32_t* seq, int32_t n) {
  return la_seed_pool_seq(c, 0, seq, n);
}

la_status la_seed_pool_seq(la_ctx* c, int32_t sq, const int32_t* seq, int32_t n) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  const la_config& g = c->cfg;
  if (sq < 0 || sq >= c->B) return fail(c, LA_ERR_INVALID_ARG, "sequence index out of range");
  if (n < 0 || (n > 0 && !seq)) return fail(c, LA_ERR_INVALID_ARG, "seq/n");
  for (int i = 0; i < n; i++)
    if (seq[i] < 0 || seq[i] >= g.vocab) return fail(c, LA_ERR_INVALID_ARG, "token out of range");
  if (!c->prefilled[sq]) return fail(c, LA_ERR_STATE, "la_seed_pool before la_prefill");
  const int n1 = g.N - 1;
  if (g.G == 0 || n <= n1) return LA_OK;
  LA_HIP(c, hipStreamSynchronize(c->stream));
  // chunks of MR tokens overlapping by N-1, so every n-gram lies in one chunk
  for (int p0 = 0; p0 + n1 < n; p0 += c->MR - n1) {
    const int m = std::min(c->MR, n - p0);
    memcpy(c->pin, seq + p0, sizeof(int32_t) * m);
    LA_HIP(c, hipMemcpyAsync(c->prompt_buf, c->pin, sizeof(int32_t) * m, hipMemcpyHostToDevice,
                             c->stream));
    launch_seed_pool(c->prompt_buf, m, c->pool_len + (size_t)sq * g.vocab, c->pool + sq * c->pool_seq,
                     g.N, g.G, c->stream);
    LA_HIP(c, hipGetLastError());
    LA_HIP(c, hipStreamSynchronize(c->stream));
  }
  return LA_OK;
}

la_status la_debug_pool_insert(la_ctx* c, int32_t key, const int32_t* tail) {
  return la_debug_pool_insert_seq(c, 0, key, tail);
}

la_status la_debug_pool_insert_seq(la_ctx* c, int32_t sq, int32_t key, const int32_t* tail) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  const la_config& g = c->cfg;
  if (sq < 0 || sq >= c->B) return fail(c, LA_ERR_INVALID_ARG, "sequence index out of range");
  if (!tail || key < 0 || key >= g.vocab) return fail(c, LA_ERR_INVALID_ARG, "key/tail");
  for (int i = 0; i < g.N - 1; i++)
    if (tail[i] < 0 || tail[i] >= g.vocab) return fail(c, LA_ERR_INVALID_ARG, "tail token out of range");
  LA_HIP(c, hipStreamSynchronize(c->stream));
  memcpy(c->pin, tail, sizeof(int32_t) * (g.N - 1));
  LA_HIP(c, hipMemcpyAsync(c->tail_buf, c->pin, sizeof(int32_t) * (g.N - 1), hipMemcpyHostToDevice,
                           c->stream));
  launch_pool_insert(c->st + sq, key, c->tail_buf, c->pool_len + (size_t)sq * g.vocab,
                     c->pool + sq * c->pool_seq, g.N, g.G, c->stream);
  LA_HIP(c, hipGetLastError());
  LA_HIP(c, hipStreamSynchronize(c->stream));
  return LA_OK;
}

la_status la_debug_kv(la_ctx* c, int32_t layer, int32_t pos0, int32_t n, float* k, float* v) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  const la_config& g = c->cfg;
  if (layer < 0 || layer >= g.n_layers || pos0 < 0 || n < 0 || pos0 + n > g.max_ctx || !k || !v)
    return fail(c, LA_ERR_INVALID_ARG, "kv range");
  LA_HIP(c, hipStreamSynchronize(c->stream));
  const int dh = g.head_dim, Hkv = g.n_kv_heads, es = c->elem;
  std::vector<char> kb((size_t)n * dh * es), vb((size_t)dh * n * es);
  // sequence b's kv head hk is head b * Hkv + hk of the layer's cache
  for (int h = 0; h < Hkv * c->B; h++) {
    const char* ks = (const char*)layer_k(c, layer) + (((size_t)h * c->ctx_stride + pos0) * dh) * es;
    LA_HIP(c, hipMemcpy(kb.data(), ks, kb.size(), hipMemcpyDeviceToHost));
    const char* vs = (const char*)layer_v(c, layer) + ((size_t)h * dh * c->ctx_stride + pos0) * es;
    LA_HIP(c, hipMemcpy2D(vb.data(), (size_t)n * es, vs, (size_t)c->ctx_stride * es, (size_t)n * es, dh,
                          hipMemcpyDeviceToHost));
    for (int p = 0; p < n; p++)
      for (int i = 0; i < dh; i++) {
        size_t o = ((size_t)h * n + p) * dh + i;
        size_t ki = (size_t)p * dh + i, vi = (size_t)i * n + p;
        if (es == 2) {
          k[o] = bf2f(((const uint16_t*)kb.data())[ki]);
          v[o] = bf2f(((const uint16_t*)vb.data())[vi]);
        } else {
          k[o] = ((const float*)kb.data())[ki];
          v[o] = ((const float*)vb.data())[vi];
        }
      }
  }
  return LA_OK;
}

la_status la_debug_state(la_ctx* c, int32_t* kv_len, int32_t* current) {
  la_status us = check_usable(c);
  if (us != LA_OK) return us;
  std::vector<DevState> hs(c->B);
  LA_HIP(c, hipStreamSynchronize(c->stream));
  LA_HIP(c, hipMemcpy(hs.data(), c->st, sizeof(DevState) * c->B, hipMemcpyDeviceToHost));
  for (int b = 0; b < c->B; b++) {
    if (kv_len) kv_len[b] = hs[b].L;
    if (current) current[b] = hs[b].cur;
  }
  return LA_OK;
}

size_t la_attention_workspace_bytes(int32_t n_heads, int32_t head_dim, int32_t ctx_stride, int32_t W,
                                    int32_t N, int32_t G) {
  if (n_heads < 1 || head_dim != 128 || ctx_stride < 1 || N < 2 || W < 0 || G < 0) return 0;
  const int T = 1 + (W + G) * (N - 1);
  if (T > MAX_ROWS) return 0;
  const int splits = attn_bf16_splits(n_heads, T, ctx_stride);
  const size_t rows = (size_t)n_heads * splits * ((T + 15) & ~15);
  return align_up(rows * head_dim * 4, 256) + align_up(rows * 2 * 4, 256);
}

namespace {

// Host-side checks of one kernel-level attention call (no HIP call).
la_status attention_check(const void* q, const void* k_cache, const void* vt_cache, const void* out,
                          int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                          int32_t prefix_len, int32_t ctx_stride, int32_t W, int32_t N, int32_t G) {
  if (!q || !k_cache || !vt_cache || !out) return LA_ERR_INVALID_ARG;
  if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads || N < 2 || N > 32 || W < 0 || G < 0 ||
      prefix_len < 0 || ctx_stride < 1)
    return LA_ERR_INVALID_ARG;
  if (head_dim != 128 || ctx_stride > (1 << 24)) return LA_ERR_UNSUPPORTED;
  const long T = 1 + (long)(W + G) * (N - 1);
  if (T > MAX_ROWS) return LA_ERR_UNSUPPORTED;
  if (ctx_stride % 64 || prefix_len + T > ctx_stride) return LA_ERR_INVALID_ARG;
  return LA_OK;
}

// Launch one checked call with the split-KV partials (if the launch uses
// any) in ws.
la_status attention_launch(const void* q, const void* k_cache, const void* vt_cache, void* out,
                           int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                           int32_t prefix_len, int32_t ctx_stride, int32_t W, int32_t N, int32_t G,
                           void* ws, void* stream) {
  const int T = 1 + (W + G) * (N - 1);
  AttnArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.splits = attn_bf16_splits(n_heads, T, ctx_stride);
  const size_t rows = (size_t)n_heads * aa.splits * ((T + 15) & ~15);
  aa.part_o = (float*)ws;
  aa.part_ml = (float*)((char*)ws + align_up(rows * head_dim * 4, 256));
  aa.q = q;
  aa.k_cache = k_cache;
  aa.vt_cache = vt_cache;
  aa.out = out;
  aa.out_mtt = 0;
  aa.st = nullptr;
  aa.L_host = prefix_len;
  aa.M = T;
  aa.rps = T;
  aa.nseq = 1;
  aa.kv_seq = 0;
  aa.mode = MODE_STEP;
  aa.H = n_heads;
  aa.Hkv = n_kv_heads;
  aa.dh = head_dim;
  aa.ctx_stride = ctx_stride;
  aa.W = W;
  aa.N = N;
  launch_attn_bf16(aa, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // namespace

la_status la_attention(const void* q, const void* k_cache, const void* vt_cache, void* out,
                       int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t prefix_len,
                       int32_t ctx_stride, int32_t W, int32_t N, int32_t G, void* workspace,
                       size_t workspace_bytes, void* stream) {
  const la_status st = attention_check(q, k_cache, vt_cache, out, n_heads, n_kv_heads, head_dim,
                                       prefix_len, ctx_stride, W, N, G);
  if (st != LA_OK) return st;
  const size_t need = la_attention_workspace_bytes(n_heads, head_dim, ctx_stride, W, N, G);
  if (!workspace || workspace_bytes < need) return LA_ERR_OUT_OF_CAPACITY;
  return attention_launch(q, k_cache, vt_cache, out, n_heads, n_kv_heads, head_dim, prefix_len,
                          ctx_stride, W, N, G, workspace, stream);
}

// ---- kernel-level attention without a caller workspace -----------------
// The split-KV partials of la_attention_noalloc live in this file-scope
// device array: one copy per GPU, held until the process ends.  On the
// host the array's name is only a stand-in, never a device address: host
// code takes the address hipGetSymbolAddress gives for the current device,
// once per device, and passes that.
static __device__ __align__(256) unsigned char scratch[LA_ATTENTION_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
constexpr int SCRATCH_MAX_DEVICES = 64;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES];

// This device's copy of `scratch` (resolved on the device's first call).
la_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return LA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LA_OK;
}
}  // namespace

la_status la_attention_noalloc(const void* q, const void* k_cache, const void* vt_cache, void* out,
                               int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                               int32_t prefix_len, int32_t ctx_stride, int32_t W, int32_t N,
                               int32_t G, void* stream) {
  la_status st = attention_check(q, k_cache, vt_cache, out, n_heads, n_kv_heads, head_dim,
                                 prefix_len, ctx_stride, W, N, G);
  if (st != LA_OK) return st;
  if (la_attention_workspace_bytes(n_heads, head_dim, ctx_stride, W, N, G) >
      LA_ATTENTION_NOALLOC_SCRATCH_BYTES)
    return LA_ERR_OUT_OF_CAPACITY;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != LA_OK) return st;
  return attention_launch(q, k_cache, vt_cache, out, n_heads, n_kv_heads, head_dim, prefix_len,
                          ctx_stride, W, N, G, ws, stream);
}

la_status la_sample(const float* logits, int32_t rows, int32_t vocab, float temperature,
                    int32_t top_k, float top_p, uint64_t seed, const int64_t* positions,
                    int32_t* out, void* stream) {
  if (!logits || !positions || !out || rows < 0 || vocab < 1) return LA_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !std::isfinite(temperature) || top_k < 0 ||
      !(top_p > 0.f && top_p <= 1.f))
    return LA_ERR_INVALID_ARG;
  if (vocab > SAMPLE_MAX_VOCAB) return LA_ERR_UNSUPPORTED;
  if (rows == 0) return LA_OK;
  SampleParams p;
  memset(&p, 0, sizeof(p));
  p.temperature = temperature;
  p.top_k = top_k;
  p.top_p = top_p;
  p.seed_lo = (uint32_t)seed;
  p.seed_hi = (uint32_t)(seed >> 32);
  launch_sample_rows(logits, rows, vocab, p, positions, out, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"
