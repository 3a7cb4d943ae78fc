// Masked attention of the lookahead step: every block row attends to the
// whole committed cache and to the block rows the lookahead/verification
// mask lets it see ("Break the Sequential Dependency of LLM Inference Using
// Lookahead Decoding", Summary: lookahead and verification branches share
// one forward pass; the method works with FlashAttention-style kernels).
//
// bf16 kernel (gfx950, head_dim 128):
//   - grid = heads x (KV splits x row groups) x sequences (flash-decoding
//     style split of the key range so short contexts still fill the CUs;
//     each sequence of a batch attends to its own cache only); a workgroup
//     holds 32 NRP query rows of its head (NRP row pairs of 16-row tiles),
//     and the row groups of one head and split read the same K/V chunks
//     (from HBM once, then from L2: their workgroup ids differ by a
//     multiple of the head count, so they land on the same XCD);
//   - Q and 64-key chunks of K and V^T go straight from HBM into LDS
//     (global_load_lds), XOR-swizzled so the MFMA operand reads are free of
//     bank conflicts, through a ring of chunk buffers a few chunks deep;
//   - S^T = K Q^T on MFMA, so a lane owns one token's scores; the block mask
//     is computed per row as a 256-bit set (closed form of the mask), and
//     chunks wholly inside the committed prefix skip it;
//   - O^T = V^T P^T on MFMA: P^T feeds MFMA straight from the score
//     registers (keys are assigned to score rows so that the 8 keys a lane
//     passes on are one contiguous V^T piece);
//   - splits merge in a second kernel (log-sum-exp weights).
// The cache stores V transposed ([kv head][dh][position]) for this reason.
#include <algorithm>
#include <type_traits>

#include "la_epilogue.h"

namespace la {

constexpr int AKC = 64;        // keys per chunk
constexpr int A_DH = 128;      // head_dim of the bf16 kernel
constexpr float LOG2E = 1.4426950408889634f;

// Max / sum over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48), with the gfx950 row swaps instead of LDS permutes:
// permlane16_swap(v, v) yields rows (0, 0, 2, 2) and (1, 1, 3, 3) of v,
// permlane32_swap(v, v) halves (0, 0) and (1, 1); combining each pair gives
// every lane the same operands, in the same order, as xor-16 then xor-32
// shuffles would.
__device__ inline float swap_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float wave_max_groups(float v) {
  v = swap_max16(v);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float wave_sum_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Visible keys of one 64-key chunk for one query row, as a bit per key
// (bit o: key at block index b0 + o).  Keys before the block (b < 0) are
// the committed cache, always visible; keys past the block are never.
//   causal: block row t sees block rows <= t;
//   step:   rm0..rm3 hold the row's 256-bit block mask.
__device__ inline uint64_t chunk_window(bool causal, int t, int b0, uint64_t rm0, uint64_t rm1,
                                        uint64_t rm2, uint64_t rm3) {
  if (causal) {
    const int tl = t - b0;  // keys o <= tl visible
    return tl >= 63 ? ~0ull : (tl < 0 ? 0ull : ((2ull << tl) - 1ull));
  }
  if (b0 < 0) {  // -63 <= b0 < 0 for a chunk that reaches into the block
    const int n = -b0;
    return (rm0 << n) | ((1ull << n) - 1ull);
  }
  const int wi = b0 >> 6, sh = b0 & 63;
  const uint64_t lo = wi == 0 ? rm0 : wi == 1 ? rm1 : wi == 2 ? rm2 : wi == 3 ? rm3 : 0ull;
  const uint64_t hi = wi == 0 ? rm1 : wi == 1 ? rm2 : wi == 2 ? rm3 : 0ull;
  return sh ? (lo >> sh) | (hi << (64 - sh)) : lo;
}

// Bits [lo, hi) of word wi (bits 64 wi .. 64 wi + 63) of a 256-bit mask.
__device__ inline uint64_t range_bits(int wi, int lo, int hi) {
  const int a = max(lo - 64 * wi, 0), b = min(hi - 64 * wi, 64);
  if (a >= b) return 0ull;
  const uint64_t upto = b == 64 ? ~0ull : ((1ull << b) - 1ull);
  return upto & ~((1ull << a) - 1ull);
}

// The block rows that step-layout row t sees, as a 256-bit mask m0..m3
// (the same relation as row_sees, in closed form): every row sees row 0; a
// window row (level l, column j) sees level-1 columns 0..j and its own
// column at levels 2..l; candidate row (g, i) sees (g, 1..i).
__device__ inline void step_row_mask(int t, int W, int N, uint64_t& m0, uint64_t& m1,
                                     uint64_t& m2, uint64_t& m3) {
  const RowDesc d = row_desc(t, W, N);
  int lo = 0, hi = 1;  // one contiguous run besides row 0
  if (d.kind == 1) { lo = 1; hi = d.b + 2; }
  if (d.kind == 2) { lo = 1 + (N - 1) * W + d.a * (N - 1); hi = lo + d.b; }
  m0 = range_bits(0, lo, hi) | 1ull;
  m1 = range_bits(1, lo, hi);
  m2 = range_bits(2, lo, hi);
  m3 = range_bits(3, lo, hi);
  if (d.kind == 1)
    for (int lv = 2; lv <= d.a; lv++) {
      const int b = 1 + (lv - 1) * W + d.b;
      const uint64_t bit = 1ull << (b & 63);
      const int wi = b >> 6;
      m0 |= wi == 0 ? bit : 0ull;
      m1 |= wi == 1 ? bit : 0ull;
      m2 |= wi == 2 ? bit : 0ull;
      m3 |= wi == 3 ? bit : 0ull;
    }
}

// LDS chunk layouts (16-byte pieces, XOR-swizzled so that the MFMA operand
// reads below hit 16 distinct bank groups):
//   K:   key r (0..63) owns bytes [256 r, 256 r + 256); dims 8p..8p+7 sit in
//        slot p ^ kswz(r);
//   V^T: dim d (0..127) owns bytes [128 d, 128 d + 128); keys 8p..8p+7 sit
//        in slot p ^ ((d >> 1) & 7).
__device__ inline int kswz(int r) { return ((r >> 1) & 12) | (r & 3); }
constexpr int CH_K_BYTES = AKC * A_DH * 2;  // 16 KiB
constexpr int CH_BYTES = 2 * CH_K_BYTES;    // K + V^T

// Score tile kt (0..3), row r (0..15) holds key 32(kt/2) + 8(r/4) + 4(kt%2)
// + r%4 of the chunk.  With this order the P^T operand a lane passes to the
// PV MFMA (tiles 2 s2 and 2 s2 + 1, rows 4g..4g+3) covers keys
// 32 s2 + 8g .. 32 s2 + 8g + 7, one contiguous V^T piece.
__device__ inline int score_key(int kt, int r) {
  return 32 * (kt >> 1) + 8 * (r >> 2) + 4 * (kt & 1) + (r & 3);
}

// Softmax reference maxima move only when a score exceeds the current one by
// more than 2^RESCALE_LOG2: probabilities relative to a stale maximum stay
// below 2^RESCALE_LOG2 (exact in fp32 sums, same relative precision in
// bf16), and the rescaling of the output accumulators is rarely needed.
constexpr float RESCALE_LOG2 = 8.f;

// One workgroup = one head x one range of 64-key chunks x 32 NRP query rows
// (row group rg: rows 32 NRP rg ..).
// NRP x KSPL waves: wave w owns 16-row tiles 2 rp and 2 rp + 1 (rp = w %
// NRP), so every K / V^T fragment read from LDS feeds two MFMAs, and key
// part kp = w / NRP of each chunk (KSPL parts); the key parts are merged
// through LDS at the end.  Chunks go straight from HBM to LDS
// (global_load_lds, no register staging) through a ring of NBUF buffers,
// NBUF - 1 chunks ahead of the one being consumed.
// Key splits used for M block rows over nch 64-key chunks (context +
// block), chosen at run time from the committed length so one captured
// graph fits every length, at most smax (the launch's grid and the partial
// buffers).  Up to 16 rows (one-token decode) a workgroup's chunk work is
// small next to its fixed costs: one or two chunks per split, up to 8
// splits.  Larger blocks: about three chunks per split, and one split (no
// merge) for two chunks or fewer.  Measured, 32 heads, in captured graphs:
// 1 row: 6 splits best at 5 and 9 chunks, 8 at 16; 121 rows: 1 split at 2
// chunks, 2-3 at 6, 3-4 at 11, 4 at 18.
__host__ __device__ inline int eff_splits(int nch, int smax, int M) {
  const int s = M <= 16 ? (nch < 8 ? nch : 8) : (nch <= 2 ? 1 : (nch + 2) / 3);
  return s < smax ? s : smax;
}

template <int NRP, int KSPL, int NBUF>
__global__ __launch_bounds__(NRP * KSPL * 64) void k_attn_bf16(AttnArgs a) {
  constexpr int NW = NRP * KSPL;
  constexpr int QROWS = 32 * NRP;                // query rows held
  constexpr int QPT = QROWS * 256 / 1024 / NW;   // Q load instructions per thread
  constexpr int LPC = 32 / NW;                   // chunk load instructions per thread
  constexpr int KT = 4 / KSPL;                   // 16-key score tiles per wave and chunk
  static_assert(QPT * NW * 1024 == QROWS * 256 && LPC * NW == 32 && KT * KSPL == 4, "shape");
  static_assert(KSPL == 1 || NBUF * CH_BYTES >= NRP * 2 * 8 * 64 * 16 + NRP * 2 * 64 * 8,
                "key-part exchange fits in the ring");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NBUF * CH_BYTES + QROWS * 256];

  const int M = a.M;
  const int RG = (M + QROWS - 1) / QROWS;  // row groups
  const int h = blockIdx.x, sq = blockIdx.z;  // head, sequence
  const int sp = blockIdx.y / RG, tb = (blockIdx.y % RG) * QROWS;  // key split, first row
  // the wave index is wave-uniform: LDS destinations and chunk bases go to scalar registers
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63,
            g = l >> 4, c16 = l & 15;
  const int rp = w % NRP, kp = w / NRP;
  const int r0 = sq * a.rps;  // the sequence's first row in q and out

  // Q of the group's rows: local row t (0 .. QROWS - 1, row tb + t; padding
  // rows repeat row M - 1) owns bytes [256 t, 256 t + 256) after the chunk
  // ring; dims 8p..8p+7 sit in slot p ^ (t & 15).
  unsigned char* qb = lds + NBUF * CH_BYTES;
#pragma unroll
  for (int q = 0; q < QPT; q++) {
    const int j = w + q * NW;  // 1 KiB = 4 rows
    const int t = 4 * j + (l >> 4), qs = l & 15;
    const uint16_t* gq = (const uint16_t*)a.q + (size_t)(r0 + min(tb + t, M - 1)) * (a.H * A_DH) +
                         h * A_DH + ((qs ^ (t & 15)) * 8);
    __builtin_amdgcn_global_load_lds((const void*)gq,
                                     (__attribute__((address_space(3))) void*)(qb + j * 1024), 16,
                                     0, 0);
  }

  // The committed length, read while the Q loads are in flight: a scalar
  // load (constant address space; nothing writes the state during this
  // kernel), so waiting for it does not wait for Q.
  const int L = a.st ? *(const __attribute__((address_space(4))) int32_t*)&a.st[sq].L : a.L_host;
  const int kvh = (h * a.Hkv) / a.H;
  const int ctx = L + M;
  const int nch = (ctx + AKC - 1) / AKC;
  const int S = eff_splits(nch, a.splits, M);
  if (sp >= S) {  // a split this length does not use (uniform)
    wait_vm<0>();   // Q loads land before the LDS is released
    return;
  }
  const int cps = (nch + S - 1) / S;
  const int c0 = min(sp * cps, nch), c1 = min(nch, c0 + cps);
  const int nloc = c1 - c0;
  const int rows16 = (M + 15) & ~15;
  const float sl2 = LOG2E / sqrtf((float)A_DH);
  const bool causal = a.mode == MODE_CAUSAL;

  const uint16_t* kc = (const uint16_t*)a.k_cache + sq * a.kv_seq + (size_t)kvh * a.ctx_stride * A_DH;
  const uint16_t* vc = (const uint16_t*)a.vt_cache + sq * a.kv_seq + (size_t)kvh * A_DH * a.ctx_stride;

  // Rows of this wave's two tiles (padding tokens take a valid row).
  int trow[2];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int t = tb + (2 * rp + u) * 16 + c16;
    trow[u] = t < M ? t : (causal ? M - 1 : 0);
  }
  const bool act = tb + 2 * rp * 16 < M;  // tile 2 rp holds tokens
  const bool act1 = tb + (2 * rp + 1) * 16 < M;

  // Issue chunk c into ring slot b.  Instruction j of a chunk (wave-uniform
  // LDS base, 1 KiB per instruction) covers K keys 4j..4j+3 or V^T dims
  // 8j..8j+7; lane l loads the global piece that belongs at LDS slot l.  The
  // lane's byte offsets within a chunk are fixed (32-bit: the V^T rows of one
  // head span 128 x ctx_stride x 2 bytes, ctx_stride <= 2^24); the chunk's
  // own offset is wave-uniform.
  uint32_t koff[LPC / 2], voff[LPC / 2];
#pragma unroll
  for (int q = 0; q < LPC / 2; q++) {
    const int j = w + q * NW;  // 0..15
    const int r = 4 * j + (l >> 4), sk = l & 15;
    koff[q] = (uint32_t)(r * A_DH + ((sk ^ kswz(r)) * 8)) * 2u;
    const int d = 8 * j + (l >> 3), sv = l & 7;
    voff[q] = ((uint32_t)d * (uint32_t)a.ctx_stride + (uint32_t)((sv ^ ((d >> 1) & 7)) * 8)) * 2u;
  }
  auto issue = [&](int c, int b) {
    c = min(c, nch - 1);  // an empty range (c0 == nch) stages a valid chunk
    unsigned char* kb = lds + b * CH_BYTES;
    unsigned char* vb = kb + CH_K_BYTES;
    const unsigned char* kg = (const unsigned char*)(kc + (size_t)c * AKC * A_DH);
    const unsigned char* vg = (const unsigned char*)(vc + (size_t)c * AKC);
#pragma unroll
    for (int q = 0; q < LPC / 2; q++) {
      const int j = w + q * NW;
      __builtin_amdgcn_global_load_lds((const void*)(kg + koff[q]),
                                       (__attribute__((address_space(3))) void*)(kb + j * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vg + voff[q]),
                                       (__attribute__((address_space(3))) void*)(vb + j * 1024),
                                       16, 0, 0);
    }
  };

  // prologue: the first NBUF - 1 chunks (chunk indices clamped so that an
  // empty or short range still issues the same count of loads)
#pragma unroll
  for (int i = 0; i < NBUF - 1; i++) issue(c0 + min(i, max(nloc - 1, 0)), i);
  wait_vm<(NBUF - 2) * LPC>();  // Q (issued first) has landed
  lds_barrier();
  bf16x8 qf[2][4];  // Q fragments of this wave's tiles, held for the whole loop
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int t = (2 * rp + u) * 16 + c16;
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
      qf[u][ks] = *(const bf16x8*)(qb + t * 256 + (((4 * ks + g) ^ c16) << 4));
  }

  f32x4 o[2][8];
  float m_run[2], l_run[2];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) o[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One 64-key chunk for this wave's tiles: TWO = the second tile holds
  // rows (else its MFMAs and softmax are skipped), MASKED = the chunk reaches
  // into the block (else every key is committed prefix, visible to every
  // row, and lies inside the context).  Scores stay unscaled until the
  // exponent: max(s) * scale is the max of the scaled scores (rounding is
  // monotone), and exp2(s * scale - m) is one fma.
  auto chunk = [&](auto two, auto masked, const unsigned char* kb, const unsigned char* vb,
                   int c) {
    constexpr bool TWO = decltype(two)::value, MASKED = decltype(masked)::value;
    f32x4 s[2][KT];
#pragma unroll
    for (int j = 0; j < KT; j++) {
      const int kt = kp * KT + j;
      s[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[1][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = score_key(kt, c16);
      const unsigned char* krow = kb + r * 256;
      const int sw = kswz(r);
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        const bf16x8 kf = *(const bf16x8*)(krow + (((4 * ks + g) ^ sw) << 4));
        s[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], s[0][j], 0, 0, 0);
        if constexpr (TWO)
          s[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], s[1][j], 0, 0, 0);
      }
    }
    bf16x8 pf[2][KT / 2];
#pragma unroll
    for (int u = 0; u < (TWO ? 2 : 1); u++) {
      if constexpr (MASKED) {  // the row's 256-bit block mask, recomputed (few chunks are masked)
        uint64_t rm0 = 0ull, rm1 = 0ull, rm2 = 0ull, rm3 = 0ull;
        if (!causal) step_row_mask(trow[u], a.W, a.N, rm0, rm1, rm2, rm3);
        const uint64_t win = chunk_window(causal, trow[u], c * AKC - L, rm0, rm1, rm2, rm3) >> (8 * g);
#pragma unroll
        for (int j = 0; j < KT; j++) {
          const int kt = kp * KT + j;
#pragma unroll
          for (int v = 0; v < 4; v++) {
            const int bit = 32 * (kt >> 1) + 4 * (kt & 1) + v;
            if (!((win >> bit) & 1ull)) s[u][j][v] = -INFINITY;
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < KT; j++)
#pragma unroll
        for (int v = 0; v < 4; v++) mx = fmaxf(mx, s[u][j][v]);
      mx = wave_max_groups(mx) * sl2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run[u] + RESCALE_LOG2)) {  // wave-uniform
        const float m_new = fmaxf(m_run[u], mx);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[u] - m_new);
        l_run[u] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; d++) o[u][d] *= alpha;
        m_run[u] = m_new;
      }
      const float nm = m_run[u] == -INFINITY ? 0.f : -m_run[u];  // nothing visible yet: 0
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < KT; j++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[u][j][v], sl2, nm));
          s[u][j][v] = p;
          ps += p;
        }
      l_run[u] += ps;
#pragma unroll
      for (int j2 = 0; j2 < KT / 2; j2++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          pf[u][j2][v] = (__bf16)s[u][2 * j2][v];
          pf[u][j2][4 + v] = (__bf16)s[u][2 * j2 + 1][v];
        }
    }
    // O^T += V^T P^T over this wave's 32-key steps.  Keys past ctx (last
    // chunk only, a masked one) have zero probability, but their V^T entries
    // may be stale or uninitialised memory: mask them to zero so that no NaN
    // reaches the MFMA.
    const int nvk = ctx - c * AKC;
#pragma unroll
    for (int j2 = 0; j2 < KT / 2; j2++) {
      const int s2 = kp * (KT / 2) + j2;
      const int kv = nvk - (32 * s2 + 8 * g);  // valid keys among this lane's 8
      const uint32_t vm0 = kv >= 2 ? ~0u : (kv == 1 ? 0xffffu : 0u);
      const uint32_t vm1 = kv >= 4 ? ~0u : (kv == 3 ? 0xffffu : 0u);
      const uint32_t vm2 = kv >= 6 ? ~0u : (kv == 5 ? 0xffffu : 0u);
      const uint32_t vm3 = kv >= 8 ? ~0u : (kv == 7 ? 0xffffu : 0u);
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const int d = dt * 16 + c16;
        bf16x8 vf = *(const bf16x8*)(vb + d * 128 + (((4 * s2 + g) ^ ((d >> 1) & 7)) << 4));
        if constexpr (MASKED) {
          if (!a.vt_finite && nvk < AKC) {  // uniform
            uint4 vr = __builtin_bit_cast(uint4, vf);
            vr.x &= vm0; vr.y &= vm1; vr.z &= vm2; vr.w &= vm3;
            vf = __builtin_bit_cast(bf16x8, vr);
          }
        }
        o[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[0][j2], o[0][dt], 0, 0, 0);
        if constexpr (TWO)
          o[1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[1][j2], o[1][dt], 0, 0, 0);
      }
    }
  };

  // The chunk loop, one copy per tile count (WORK: 2 = both tiles hold rows,
  // 1 = the first only, 0 = neither: the wave only loads and meets the
  // barriers), and within it one run over the chunks wholly inside the
  // committed prefix (no mask) followed by one over those reaching into the
  // block, so no branch on either sits inside a loop.
  const int nfree = min(max(L / AKC - c0, 0), nloc);  // chunks c0 .. c0 + nfree - 1 need no mask
  auto step = [&](int i, auto work, auto masked) {
    constexpr int WORK = decltype(work)::value;
    // keep NBUF - 1 chunks in flight: chunk i + NBUF - 1 goes into the slot
    // chunk i - 1 used (every wave finished with it at the last barrier);
    // past the end the last chunk is re-issued, never read
    issue(c0 + min(i + NBUF - 1, nloc - 1), (i + NBUF - 1) % NBUF);
    wait_vm<(NBUF - 1) * LPC>();  // this thread's part of chunk i has landed
    lds_barrier();                 // ... and everyone else's
    if constexpr (WORK > 0) {
      const unsigned char* kb = lds + (i % NBUF) * CH_BYTES;
      chunk(std::integral_constant<bool, WORK == 2>{}, masked, kb, kb + CH_K_BYTES, c0 + i);
    }
    lds_barrier();  // slot i % NBUF is free for the next issue
  };
  auto run = [&](auto work) {
    int i = 0;
    for (; i < nfree; i++) step(i, work, std::false_type{});
    for (; i < nloc; i++) step(i, work, std::true_type{});
  };
  if (act1)
    run(std::integral_constant<int, 2>{});
  else if (act)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 0>{});
  wait_vm<0>();  // drain the ring's redundant loads (also before LDS reuse)

  float lsum[2];
#pragma unroll
  for (int u = 0; u < 2; u++) lsum[u] = wave_sum_groups(l_run[u]);

  if constexpr (KSPL == 2) {
    // key part 1 hands (m, l, O) to key part 0 through the (idle) ring
    lds_barrier();
    f32x4* xo = (f32x4*)lds;                                     // [rp][u][dt][lane]
    float* xm = (float*)(lds + NRP * 2 * 8 * 64 * 16);           // [rp][u][lane][2]
    if (kp == 1) {
#pragma unroll
      for (int u = 0; u < 2; u++) {
#pragma unroll
        for (int dt = 0; dt < 8; dt++) xo[((rp * 2 + u) * 8 + dt) * 64 + l] = o[u][dt];
        xm[((rp * 2 + u) * 64 + l) * 2] = m_run[u];
        xm[((rp * 2 + u) * 64 + l) * 2 + 1] = lsum[u];
      }
    }
    lds_barrier();
    if (kp == 1) return;
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const float mb = xm[((rp * 2 + u) * 64 + l) * 2], lb = xm[((rp * 2 + u) * 64 + l) * 2 + 1];
      const float ms = fmaxf(m_run[u], mb);
      const float wa = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[u] - ms);
      const float wb = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb - ms);
      lsum[u] = wa * lsum[u] + wb * lb;
#pragma unroll
      for (int dt = 0; dt < 8; dt++) o[u][dt] = wa * o[u][dt] + wb * xo[((rp * 2 + u) * 8 + dt) * 64 + l];
      m_run[u] = ms;
    }
  }

  if (!act) return;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    if (u == 1 && !act1) break;
    const int t = tb + (2 * rp + u) * 16 + c16;
    if (t >= M) continue;
    if (S == 1) {
      // row-major, or fragment layout (dims dt*16 + 4g + 0..3 stay adjacent)
      uint16_t* out = (uint16_t*)a.out;
      const float inv = 1.f / lsum[u];
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const int k = h * A_DH + dt * 16 + 4 * g;
        const size_t o0 = a.out_mtt ? frag_index(r0 + t, k, a.out_mtt) : (size_t)(r0 + t) * (a.H * A_DH) + k;
        uint2 pk;
        pk.x = (uint32_t)f2bf(o[u][dt][0] * inv) | ((uint32_t)f2bf(o[u][dt][1] * inv) << 16);
        pk.y = (uint32_t)f2bf(o[u][dt][2] * inv) | ((uint32_t)f2bf(o[u][dt][3] * inv) << 16);
        *(uint2*)&out[o0] = pk;
      }
    } else {
      float* po = a.part_o + ((((size_t)sq * a.H + h) * a.splits + sp) * rows16 + t) * A_DH;
#pragma unroll
      for (int dt = 0; dt < 8; dt++) *(f32x4*)&po[dt * 16 + 4 * g] = o[u][dt];
      if (g == 0) {
        float* pm = a.part_ml + ((((size_t)sq * a.H + h) * a.splits + sp) * rows16 + t) * 2;
        pm[0] = m_run[u];
        pm[1] = lsum[u];
      }
    }
  }
}

// Combine the splits of each (row, head) with log-sum-exp weights
// 2^(m_s - m*).  A workgroup covers 8 rows of one head of one sequence
// (grid z); a thread, 4 dims.  The (m, l, O) of every split the launch
// provides are loaded up front, together with the committed length that
// says how many of them this length used: one round trip.  The loads are
// unconditional (slots past the launch's split count repeat its last one),
// so none waits on another (a load under a per-split branch made the
// compiler wait for each before the next); slots this length did not use
// hold stale values and are not read past the load.
constexpr int A_MAX_SPLITS = 16;

__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int h = blockIdx.y, t = blockIdx.x * 8 + (threadIdx.x >> 5), i = (threadIdx.x & 31) * 4;
  const int sq = blockIdx.z;
  if (t >= a.M) return;
  const int rows16 = (a.M + 15) & ~15;
  float m[A_MAX_SPLITS], l[A_MAX_SPLITS];
  f32x4 o[A_MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < A_MAX_SPLITS; s++) {
    const size_t b = (((size_t)sq * a.H + h) * a.splits + min(s, a.splits - 1)) * rows16 + t;
    const float2 ml = *(const float2*)&a.part_ml[b * 2];
    m[s] = ml.x;
    l[s] = ml.y;
    o[s] = *(const f32x4*)&a.part_o[b * A_DH + i];
  }
  const int L = a.st ? *(const __attribute__((address_space(4))) int32_t*)&a.st[sq].L : a.L_host;
  const int S = eff_splits((L + a.M + AKC - 1) / AKC, a.splits, a.M);
  if (S == 1) return;  // one split wrote the output itself
  float mstar = -INFINITY;
#pragma unroll
  for (int s = 0; s < A_MAX_SPLITS; s++)
    if (s < S) mstar = fmaxf(mstar, m[s]);
  float den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < A_MAX_SPLITS; s++) {
    if (s < S) {
      const float wgt = (m[s] == -INFINITY) ? 0.f : exp2f(m[s] - mstar);
      den += wgt * l[s];
      num += wgt * o[s];
    }
  }
  const float inv = 1.f / den;
  const int k = h * A_DH + i;
  const int tg = sq * a.rps + t;
  const size_t oi = a.out_mtt ? frag_index(tg, k, a.out_mtt) : (size_t)tg * (a.H * A_DH) + k;
  uint2 pk;
  pk.x = (uint32_t)f2bf(num[0] * inv) | ((uint32_t)f2bf(num[1] * inv) << 16);
  pk.y = (uint32_t)f2bf(num[2] * inv) | ((uint32_t)f2bf(num[3] * inv) << 16);
  *(uint2*)&((uint16_t*)a.out)[oi] = pk;
}

// ---------------------------------------------------------------------------
// Blocks of more than 32 rows: one workgroup per (head, 16-row tile,
// sequence) that covers every key, so no split merge is needed and the
// grid (heads x tiles, 256 workgroups at 32 heads x 121 rows) fills the
// CUs by itself.  K and V^T go through LDS in 128-key chunks
// (global_load_lds, 1 KiB = 4 whole K rows or 4 whole V^T rows per
// instruction) through a ring of K and V^T slots (below); the NW = 4 waves
// share every chunk, wave w taking its keys 32 w .. 32 w + 31, and each
// runs its own online softmax over its keys; (m, l, O) of the four are
// combined through LDS at the end.  K/V of a head is read by all of its tiles' workgroups: grid x
// enumerates heads KV head first, so that the tiles of a head, and the
// query heads of one KV head, share an XCD and its L2.
constexpr int AT_NW = 4;                 // waves per workgroup
constexpr int AT_CK = 32 * AT_NW;        // keys per chunk
constexpr int AT_KB = AT_CK * A_DH * 2;  // K bytes per chunk (32 KiB), V^T as many
constexpr int AT_LPC = 2 * AT_CK / 4 / AT_NW;  // 1 KiB loads per thread per chunk (K and V^T)

// LDS V^T layout for 128-key chunks: dim d owns bytes [256 d, 256 d + 256),
// keys 8p .. 8p + 7 sit in slot p ^ (d & 15), so the 16 dims one PV operand
// read touches spread over all 64 banks.
__device__ inline int vswz16(int d) { return d & 15; }

// LDS ring: three K slots and two V^T slots of one chunk each (160 KiB,
// all of a CU's LDS).  While chunk c is consumed, K of c + 1 and c + 2 and
// V^T of c + 1 are in flight (96 KiB), half as much again as a ring of two
// whole chunks would hold.
constexpr int AT_KSLOTS = 3, AT_VSLOTS = 2;

__global__ __launch_bounds__(AT_NW * 64) void k_attn_tile(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[(AT_KSLOTS + AT_VSLOTS) * AT_KB];
  unsigned char* const vring = lds + AT_KSLOTS * AT_KB;
  const int M = a.M;
  const int gq = a.H / a.Hkv;  // query heads per KV head
  const int kvh = blockIdx.x % a.Hkv, h = kvh * gq + blockIdx.x / a.Hkv;
  const int tile = blockIdx.y, sq = blockIdx.z;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int r0 = sq * a.rps;  // the sequence's first row in q and out
  const bool causal = a.mode == MODE_CAUSAL;
  const int t = tile * 16 + c16;  // this lane's query row
  const int trow = t < M ? t : (causal ? M - 1 : 0);  // padding rows take a valid row

  bf16x8 qf[4];  // Q^T fragments of the tile (B operand), k-step ks
  {
    const uint16_t* qp = (const uint16_t*)a.q + (size_t)(r0 + trow) * (a.H * A_DH) + h * A_DH + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) qf[ks] = *(const bf16x8*)(qp + 32 * ks);
  }
  const int L = a.st ? *(const __attribute__((address_space(4))) int32_t*)&a.st[sq].L : a.L_host;
  const int ctx = L + M;
  const int nch = (ctx + AT_CK - 1) / AT_CK;
  // The tiles of a head start at different chunks (rotated by their share
  // of the chunks), so that they fetch different chunks from memory at once
  // and later find the others' chunks in L2 (measured, 32 heads x 121 rows,
  // HBM-cold: 550 keys 12.02 -> 11.64 us, 1024 keys 15.3 -> 14.6, 1900
  // keys 23.4 -> 22.2; L2-hot unchanged).  Every tile still visits its
  // chunks in one fixed order, so its result does not depend on timing.
  const int rot = (int)(((uint32_t)tile * (uint32_t)nch) / gridDim.y);
  auto chunk_of = [&](int it) { const int c = it + rot; return c < nch ? c : c - nch; };
  const float sl2 = LOG2E / sqrtf((float)A_DH);

  // Chunk loads: instruction j (of AT_LPC / 2 per thread for K, as many for
  // V^T) covers K rows 4 j' .. 4 j' + 3 or V^T dims 4 j' .. 4 j' + 3 (j' =
  // w + j NW); lane l loads the global piece that belongs at LDS slot l.
  // Keys past the cache row (the last chunk may reach 64 keys beyond
  // ctx_stride, a multiple of 64) are clamped to its last piece: they lie
  // past the context and are never used.
  const uint16_t* kc = (const uint16_t*)a.k_cache + sq * a.kv_seq + (size_t)kvh * a.ctx_stride * A_DH;
  const uint16_t* vc = (const uint16_t*)a.vt_cache + sq * a.kv_seq + (size_t)kvh * A_DH * a.ctx_stride;
  int krow[AT_LPC / 2], kpc[AT_LPC / 2], vdim[AT_LPC / 2], vkey[AT_LPC / 2];
#pragma unroll
  for (int q = 0; q < AT_LPC / 2; q++) {
    const int j = w + q * AT_NW;  // 0 .. 31
    krow[q] = 4 * j + (l >> 4);
    kpc[q] = (l & 15) ^ kswz(krow[q] & 63);
    vdim[q] = 4 * j + (l >> 4);
    vkey[q] = 8 * ((l & 15) ^ vswz16(vdim[q]));
  }
  // A chunk that lies wholly inside the cache row (every one but possibly
  // the last) is loaded from a scalar chunk base plus fixed 32-bit lane
  // offsets (the cache rows of this kernel hold at most 2048 keys, so the
  // offsets fit), which leaves no per-load address arithmetic on the VALU.
  uint32_t koff[AT_LPC / 2], voff[AT_LPC / 2];
#pragma unroll
  for (int q = 0; q < AT_LPC / 2; q++) {
    koff[q] = (uint32_t)(krow[q] * A_DH + 8 * kpc[q]) * 2u;
    voff[q] = (uint32_t)(vdim[q] * a.ctx_stride + vkey[q]) * 2u;
  }
  auto issue_k = [&](int it) {
    unsigned char* kb = lds + (it % AT_KSLOTS) * AT_KB;
    const int c = chunk_of(it);
    if ((c + 1) * AT_CK <= a.ctx_stride) {  // wave-uniform
      const char* base = (const char*)kc + (size_t)c * (AT_CK * A_DH * 2);
#pragma unroll
      for (int q = 0; q < AT_LPC / 2; q++)
        __builtin_amdgcn_global_load_lds((const void*)(base + koff[q]),
                                         (__attribute__((address_space(3))) void*)(kb + (w + q * AT_NW) * 1024),
                                         16, 0, 0);
      return;
    }
#pragma unroll
    for (int q = 0; q < AT_LPC / 2; q++) {
      const int j = w + q * AT_NW;
      const int key = min(c * AT_CK + krow[q], a.ctx_stride - 1);
      __builtin_amdgcn_global_load_lds((const void*)(kc + (size_t)key * A_DH + 8 * kpc[q]),
                                       (__attribute__((address_space(3))) void*)(kb + j * 1024),
                                       16, 0, 0);
    }
  };
  auto issue_v = [&](int it) {
    unsigned char* vb = vring + (it % AT_VSLOTS) * AT_KB;
    const int c = chunk_of(it);
    if ((c + 1) * AT_CK <= a.ctx_stride) {  // wave-uniform
      const char* base = (const char*)vc + (size_t)c * (AT_CK * 2);
#pragma unroll
      for (int q = 0; q < AT_LPC / 2; q++)
        __builtin_amdgcn_global_load_lds((const void*)(base + voff[q]),
                                         (__attribute__((address_space(3))) void*)(vb + (w + q * AT_NW) * 1024),
                                         16, 0, 0);
      return;
    }
#pragma unroll
    for (int q = 0; q < AT_LPC / 2; q++) {
      const int j = w + q * AT_NW;
      const int k0 = min(c * AT_CK + vkey[q], a.ctx_stride - 8);
      __builtin_amdgcn_global_load_lds((const void*)(vc + (size_t)vdim[q] * a.ctx_stride + k0),
                                       (__attribute__((address_space(3))) void*)(vb + j * 1024),
                                       16, 0, 0);
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // This wave's 32 keys of chunk c (slice s = 4 c + w: keys 32 s ..).  K row
  // of score-tile row c16 in tile kt: key 8 (c16 / 4) + 4 kt + c16 % 4 of
  // the slice, so that the 8 keys a lane holds after QK^T are keys
  // 8 g .. 8 g + 7, the lane's P^T operand and one contiguous V^T piece.
  // Only a slice that reaches into the block needs the mask and, if it is
  // the last one, the zeroing of V^T entries past the context; both sit in
  // one wave-uniform branch that every earlier slice (plain committed
  // cache) skips.  All K and V^T operands of the slice are read from LDS up
  // front, so their latency overlaps the MFMAs and the softmax instead of
  // stalling each pair.
  auto compute = [&](const unsigned char* kb, const unsigned char* vb, int c) {
    const int s = c * AT_NW + w;
    bf16x8 kf[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      const int r = 32 * w + 8 * (c16 >> 2) + 4 * kt + (c16 & 3);
      const unsigned char* kr = kb + r * 256;
      const int sw = kswz(r & 63);
#pragma unroll
      for (int ks = 0; ks < 4; ks++) kf[kt][ks] = *(const bf16x8*)(kr + (((4 * ks + g) ^ sw) << 4));
    }
    bf16x8 vf[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      const int d = dt * 16 + c16;
      vf[dt] = *(const bf16x8*)(vb + d * 256 + (((4 * w + g) ^ vswz16(d)) << 4));
    }
    f32x4 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ks++)
        sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][ks], qf[ks], sc[kt], 0, 0, 0);
    }
    if (32 * s + 32 > L) {  // the slice reaches into the block (wave-uniform)
      uint64_t rm0 = 0ull, rm1 = 0ull, rm2 = 0ull, rm3 = 0ull;
      if (!causal) step_row_mask(trow, a.W, a.N, rm0, rm1, rm2, rm3);
      const uint64_t win = chunk_window(causal, trow, 32 * s - L, rm0, rm1, rm2, rm3) >> (8 * g);
#pragma unroll
      for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int v = 0; v < 4; v++)
          if (!((win >> (4 * kt + v)) & 1ull)) sc[kt][v] = -INFINITY;
      // Keys past the context (last slice only) have zero probability, but
      // their V^T entries may be stale memory: unless the cache is known to
      // hold finite values there, zero them so that no NaN reaches the MFMA
      // (measured: the zeroing costs 0.35 us a call at 550 committed keys).
      if (!a.vt_finite && 32 * s + 32 > ctx) {  // wave-uniform
        const int kv = ctx - 32 * s - 8 * g;  // valid keys among this lane's 8
        const uint32_t vm0 = kv >= 2 ? ~0u : (kv == 1 ? 0xffffu : 0u);
        const uint32_t vm1 = kv >= 4 ? ~0u : (kv == 3 ? 0xffffu : 0u);
        const uint32_t vm2 = kv >= 6 ? ~0u : (kv == 5 ? 0xffffu : 0u);
        const uint32_t vm3 = kv >= 8 ? ~0u : (kv == 7 ? 0xffffu : 0u);
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
          uint4 vr = __builtin_bit_cast(uint4, vf[dt]);
          vr.x &= vm0; vr.y &= vm1; vr.z &= vm2; vr.w &= vm3;
          vf[dt] = __builtin_bit_cast(bf16x8, vr);
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int v = 0; v < 4; v++) mx = fmaxf(mx, sc[kt][v]);
    mx = wave_max_groups(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + RESCALE_LOG2)) {  // wave-uniform
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; dt++) o[dt] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == -INFINITY ? 0.f : -m_run;  // nothing visible yet: 0
    bf16x8 pf;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[kt][v], sl2, nm));
        l_run += p;
        pf[4 * kt + v] = (__bf16)p;
      }
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf, o[dt], 0, 0, 0);
  };

  // Issue order: K0 V0 K1, then per chunk c: V(c+1) K(c+2) (while they
  // exist).  The slots refilled at chunk c held chunk c - 1, finished at the
  // last barrier.  Chunk c is complete once V(c) has landed; after V(c) this
  // thread has at most K(c+1), V(c+1), K(c+2) in flight, 8 loads each.
  constexpr int G8 = AT_LPC / 2;  // loads per thread per K or V^T chunk
  issue_k(0);
  issue_v(0);
  if (nch > 1) issue_k(1);
  for (int c = 0; c < nch; c++) {
    if (c + 1 < nch) issue_v(c + 1);
    if (c + 2 < nch) issue_k(c + 2);
    if (c + 2 < nch)
      wait_vm<3 * G8>();
    else if (c + 1 < nch)
      wait_vm<2 * G8>();
    else
      wait_vm<0>();
    lds_barrier();  // every thread's part of chunk c has landed
    {
      const int cc = chunk_of(c);
      if (32 * (cc * AT_NW + w) < ctx)  // keys of this wave exist
        compute(lds + (c % AT_KSLOTS) * AT_KB, vring + (c % AT_VSLOTS) * AT_KB, cc);
    }
    lds_barrier();  // chunk c's slots may be refilled (and, after the last, the ring reused)
  }

  // combine the waves' (m, l, O) through the idle ring: wave w's O^T at
  // [w][dt][lane], its m and l per row after them
  f32x4* xo = (f32x4*)lds;
  float* xm = (float*)(lds + AT_NW * 8 * 64 * 16);
  float* xl = xm + AT_NW * 16;
  const float lsum = wave_sum_groups(l_run);
#pragma unroll
  for (int dt = 0; dt < 8; dt++) xo[(w * 8 + dt) * 64 + l] = o[dt];
  if (g == 0) {
    xm[w * 16 + c16] = m_run;
    xl[w * 16 + c16] = lsum;
  }
  __syncthreads();
  float mstar = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < AT_NW; ww++) mstar = fmaxf(mstar, xm[ww * 16 + c16]);
  float wgt[AT_NW];
  float den = 0.f;
#pragma unroll
  for (int ww = 0; ww < AT_NW; ww++) {
    const float m = xm[ww * 16 + c16];
    wgt[ww] = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mstar);
    den += wgt[ww] * xl[ww * 16 + c16];
  }
  const float inv = 1.f / den;
  if (t >= M) return;
  uint16_t* out = (uint16_t*)a.out;
  // wave w writes dim tiles w and w + 4 of the tile's rows
#pragma unroll
  for (int dt = w; dt < 8; dt += AT_NW) {
    f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < AT_NW; ww++) num += wgt[ww] * xo[(ww * 8 + dt) * 64 + l];
    const int k = h * A_DH + dt * 16 + 4 * g;
    const size_t o0 = a.out_mtt ? frag_index(r0 + t, k, a.out_mtt) : (size_t)(r0 + t) * (a.H * A_DH) + k;
    uint2 pk;
    pk.x = (uint32_t)f2bf(num[0] * inv) | ((uint32_t)f2bf(num[1] * inv) << 16);
    pk.y = (uint32_t)f2bf(num[2] * inv) | ((uint32_t)f2bf(num[3] * inv) << 16);
    *(uint2*)&out[o0] = pk;
  }
}

// Row groups of the instance launch_attn_bf16 picks for M rows: 32-row
// groups from 65 to 128 rows, one workgroup per head otherwise.
static int attn_row_groups(int M) { return M > 64 && M <= 128 ? (M + 31) / 32 : 1; }

// Waves per workgroup of that instance.
static int attn_waves(int M) { return M > 32 && M <= 64 ? 4 : (M <= 128 ? 2 : 8); }

// Splits the launch provides for (the grid's second dimension and the
// partial buffers): what eff_splits asks for at the longest context, capped
// so that up to 128 rows heads x sequences x row groups x splits x waves
// stays near 1024 waves (one per SIMD; above 128 rows near 512 workgroups):
// more splits than that only add prologues, merge traffic and waves that
// share a SIMD.  Measured in captured graphs: 40 heads x 81 rows, 1100
// committed tokens: 3-4 splits 17.8 us, 6 splits 19.2 us, 8 splits 21.4 us;
// 64 heads (8 KV heads) x 57 rows, 2100 tokens: 4 splits 20.8 us, 8 splits
// 24.2 us; 32 heads x 121 rows, 1024 tokens: 4 splits 17.5 us, 3 splits
// 19.5 us.  A large batch fills the chip without splitting the keys.  H
// counts the heads of all sequences.
int attn_bf16_splits(int H, int M, int max_ctx) {
  const int per = H * attn_row_groups(M);
  const int cap = std::max(1, M <= 128 ? 1024 / (per * attn_waves(M)) : 512 / per);
  return eff_splits((max_ctx + M + AKC - 1) / AKC, std::min(A_MAX_SPLITS, cap), M);
}


template <int NRP, int KSPL, int NBUF>
static void launch_attn_inst(const AttnArgs& a, hipStream_t s) {
  const int rg = (a.M + 32 * NRP - 1) / (32 * NRP);
  hipLaunchKernelGGL((k_attn_bf16<NRP, KSPL, NBUF>), dim3(a.H, a.splits * rg, a.nseq),
                     dim3(NRP * KSPL * 64), 0, s, a);
}

// Blocks above 32 rows take k_attn_tile (no split, no merge) while the
// cache rows are at most 2048 keys: there each CU reading the head's whole
// K/V from L2 costs less than the split kernel's extra launch and merge
// traffic, or little more at the longest contexts the capacity allows
// (the choice is fixed per launch shape, and a captured step graph serves
// every length up to ctx_stride).  Measured, HBM-cold / L2-hot, us per call
// (split + merge against k_attn_tile): 32 heads x 121 rows at 550
// committed keys 17.4 / 11.1 cold, 1024 keys 15.3 / 15.4 cold and 11.9 /
// 12.1 hot, 1536 keys 21.0 / 19.9 and 19.2 / 15.7, 2048 keys 22.4 / 24.8
// and 20.4 / 20.7, 3072 keys 27.1 / 33.8; 40 heads x 81 rows at 1100 16.7
// / 16.7, 1600 21.1 / 21.5 and 19.5 / 17.5 hot, 2400 24.5 / 28.6; 64 heads
// (8 KV heads) x 57 rows at 2100 20.6 / 21.3 and 20.6 / 18.8 hot, 4000
// 30.6 / 38.8.  The 13B-shape step (capacity 1,472 positions) takes 7.44
// ms with the split kernel and 7.32 ms with this one.
// Blocks of at most 32 rows (one-token decode, small lookahead blocks) stay
// split: with one workgroup per head (32-64 in all) each reads its head's
// whole cache, which pays only at short contexts.  Measured, 7B shape, ms
// per step (split + merge / per-tile): 128-token prompts, 1 row 2.90 /
// 2.84, an 11-row block 3.23 / 3.12, a 21-row block 3.63 / 3.39, 16 one-row
// sequences 3.62 / 3.69; 512-token prompt, 1 row 2.986 / 3.014; 13B shape,
// 1024-token prompt, 1 row: attention 0.60 / 0.74 ms per step.  Small
// blocks (one-row blocks have their own kernel) take it too while its grid
// (heads x tiles x sequences) is one or two rounds on the 256 CUs and
// either fills the first round (4 sequences of 21-row blocks, 512 /
// 1024-token prompts: 4.60 / 4.43 and 5.13 / 4.62 ms per step) or the
// cache rows are short enough that each CU reading its head's whole cache
// costs little (at most 768 keys: one 17-25-row block, 512-token prompt,
// 2% faster; at 1024-token prompts, 1216-1280-key rows, 2-4% slower).  At
// three rounds the split kernel is faster (12 sequences of 21-row blocks,
// 128 / 512-token prompts: 8.21 / 8.37 and 8.71 / 8.92).
bool attn_bf16_tiled(int M, int ctx_stride, int H, int nseq) {
  if (ctx_stride > 2048) return false;
  if (M > 32) return true;
  const int wgs = H * ((M + 15) / 16) * nseq;
  return M > 1 && wgs <= 512 && (ctx_stride <= 768 || wgs >= 256);
}

// ---------------------------------------------------------------------------
// One-row blocks (plain decode, batches of one-row sequences): the row sees
// every committed key and itself (keys 0 .. L).  A workgroup takes one
// (head, key split, sequence); its NW waves take 32-key blocks of the
// split's range in turn, loading K and V^T straight into registers (the
// next block's loads go out before the current block computes), so the
// workgroup needs LDS only for its final combine and several fit on a CU.
//
// Scores: S^T = K Q^T on 16x16x32 MFMAs, the query in every column (all 16
// columns equal), two 16-key tiles per block.  Tile u's MFMA row r holds key
// 8 (r / 4) + 4 u + r % 4, so the lane with rows 4g .. 4g+3 ends up with
// the block's keys 8g .. 8g+7 over its two tiles: exactly the key (k) range
// that lane supplies to a 16x16x32 MFMA.  Values: O^T += V^T P^T on those
// MFMAs, each lane reading 16 contiguous bytes of a V^T row (keys 8g ..
// 8g+7) and feeding its own eight probabilities as P^T.  Lazy online
// softmax per wave; the waves' (m, l, O) combine in LDS in wave order, and
// a split's result goes either to the output (one split) or to the partial
// buffers that k_attn_merge combines (the split kernel's format and split
// count, so the merge is shared).
//
// Bounds: a block starts at a multiple of 32 below the context, and the
// cache row (ctx_stride, a multiple of 32) holds the whole block.
template <int NW, bool DEEP>
__global__ __launch_bounds__(NW * 64) void k_attn_row(AttnArgs a) {
  __shared__ float xo[NW][A_DH];
  __shared__ float xm[NW], xl[NW];
  const int gq = a.H / a.Hkv;  // query heads per KV head
  // the gq heads of a KV head sit Hkv apart in the grid: with Hkv a
  // multiple of 8 their workgroups share an XCD (and its L2)
  const int kvh = blockIdx.x % a.Hkv, h = kvh * gq + blockIdx.x / a.Hkv;
  const int sp = blockIdx.y, sq = blockIdx.z;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int g = l >> 4, c16 = l & 15;
  const int r = sq * a.rps;  // the sequence's row in q and out
  const int L = a.st ? *(const __attribute__((address_space(4))) int32_t*)&a.st[sq].L : a.L_host;
  const int ctx = L + 1;
  const int S = eff_splits((ctx + AKC - 1) / AKC, a.splits, 1);
  if (sp >= S) return;  // a split this length does not use (uniform)
  const float sl2 = LOG2E / sqrtf((float)A_DH);

  bf16x8 qf[4];  // Q^T (B operand): the row's query in every column
  {
    const uint16_t* qp = (const uint16_t*)a.q + (size_t)r * (a.H * A_DH) + h * A_DH + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) qf[ks] = *(const bf16x8*)(qp + 32 * ks);
  }
  const uint16_t* kc = (const uint16_t*)a.k_cache + sq * a.kv_seq + (size_t)kvh * a.ctx_stride * A_DH;
  const uint16_t* vc = (const uint16_t*)a.vt_cache + sq * a.kv_seq + (size_t)kvh * A_DH * a.ctx_stride;
  const int nblk = (ctx + 31) / 32;  // S <= nblk: every split holds a block
  const int bs0 = nblk * sp / S, bs1 = nblk * (sp + 1) / S;

  // this lane's K row of tile u and its V^T rows, relative to the block
  const int krow = 8 * (c16 >> 2) + (c16 & 3);
  auto load = [&](bf16x8 (&kf)[2][4], bf16x8 (&vf)[8], int b) {
    const uint16_t* kb = kc + (size_t)(32 * b + krow) * A_DH + 8 * g;
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int ks = 0; ks < 4; ks++) kf[u][ks] = *(const bf16x8*)(kb + 4 * u * A_DH + 32 * ks);
    const uint16_t* vb = vc + (size_t)c16 * a.ctx_stride + 32 * b + 8 * g;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) vf[dt] = *(const bf16x8*)(vb + (size_t)(16 * dt) * a.ctx_stride);
  };
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  auto compute = [&](const bf16x8 (&kf)[2][4], bf16x8 (&vf)[8], int b) {
    f32x4 sc[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ks++)
        sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u][ks], qf[ks], sc[u], 0, 0, 0);
    }
    // sc[u][i]: key 32 b + 8 g + 4 u + i
    if (32 * b + 32 > ctx) {  // the last block (wave-uniform)
      const int kv = ctx - 32 * b - 8 * g;  // valid keys among this lane's 8
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (j >= kv) sc[j >> 2][j & 3] = -INFINITY;
      // zero the values of keys past the context (stale cache contents
      // could be NaN, and 0 x NaN is NaN) unless the cache is known to hold
      // finite values there
#pragma unroll
      for (int dt = 0; dt < 8 && !a.vt_finite; dt++) {
        uint4 vr = __builtin_bit_cast(uint4, vf[dt]);
        vr.x = kv >= 2 ? vr.x : (kv == 1 ? vr.x & 0xffffu : 0u);
        vr.y = kv >= 4 ? vr.y : (kv == 3 ? vr.y & 0xffffu : 0u);
        vr.z = kv >= 6 ? vr.z : (kv == 5 ? vr.z & 0xffffu : 0u);
        vr.w = kv >= 8 ? vr.w : (kv == 7 ? vr.w & 0xffffu : 0u);
        vf[dt] = __builtin_bit_cast(bf16x8, vr);
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = wave_max_groups(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + RESCALE_LOG2)) {  // wave-uniform
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; dt++) o[dt] *= alpha;
      m_run = m_new;
    }
    const float nm = m_run == -INFINITY ? 0.f : -m_run;
    bf16x8 pf;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[j >> 2][j & 3], sl2, nm));
      l_run += p;
      pf[j] = (__bf16)p;
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf, o[dt], 0, 0, 0);
  };
  // This wave's blocks: bs0 + w, bs0 + w + NW, ... (nb of them), through
  // two register sets.  DEEP: the loop body's loads are unconditional and
  // the last one or two blocks run after it, so the next block's loads stay
  // in flight through both products of the current one.  Otherwise the
  // block after next loads under a branch, and the compiler, counting for
  // the worst path, waits for it before the current block's value
  // products: fewer bytes in flight per wave, which measured faster once
  // the grid holds 1024 or more (head, sequence) pairs and HBM is the
  // limit (plain decode, 32 heads, 1024-token prompts, ms per step, DEEP /
  // not: batch 1 2.962 / 3.008, 16 4.742 / 4.779, 64 10.39 / 10.24, 128
  // 17.44 / 17.13).
  bf16x8 kA[2][4], kB[2][4], vA[8], vB[8];
  const int nb = bs1 - bs0 > w ? (bs1 - bs0 - w + NW - 1) / NW : 0;
  auto blk = [&](int i) { return bs0 + w + i * NW; };
  if (nb > 0) {  // wave-uniform
    load(kA, vA, blk(0));
    int i = 0;
    if constexpr (DEEP) {
      for (; i + 2 < nb; i += 2) {
        load(kB, vB, blk(i + 1));
        compute(kA, vA, blk(i));
        load(kA, vA, blk(i + 2));
        compute(kB, vB, blk(i + 1));
      }
      if (i + 1 < nb) {
        load(kB, vB, blk(i + 1));
        compute(kA, vA, blk(i));
        compute(kB, vB, blk(i + 1));
      } else {
        compute(kA, vA, blk(i));
      }
    } else {
      for (; i + 1 < nb; i += 2) {
        load(kB, vB, blk(i + 1));
        compute(kA, vA, blk(i));
        if (i + 2 < nb) load(kA, vA, blk(i + 2));
        compute(kB, vB, blk(i + 1));
      }
      if (i < nb) compute(kA, vA, blk(i));
    }
  }

  // every column holds the row; column 0 (lanes c16 = 0) is combined
  const float lsum = wave_sum_groups(l_run);
  if (c16 == 0) {
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
#pragma unroll
      for (int i = 0; i < 4; i++) xo[w][dt * 16 + 4 * g + i] = o[dt][i];
  }
  if (l == 0) {
    xm[w] = m_run;
    xl[w] = lsum;
  }
  __syncthreads();
  if (tid >= A_DH) return;
  float mstar = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < NW; ww++) mstar = fmaxf(mstar, xm[ww]);
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ww++) {
    const float wgt = xm[ww] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(xm[ww] - mstar);
    num += wgt * xo[ww][tid];
    den += wgt * xl[ww];
  }
  if (S == 1) {
    const int k = h * A_DH + tid;
    const size_t oi = a.out_mtt ? frag_index(r, k, a.out_mtt) : (size_t)r * (a.H * A_DH) + k;
    ((uint16_t*)a.out)[oi] = f2bf(num / den);
  } else {
    // the split kernel's partial layout with 16 row slots, row 0
    const size_t pb = (((size_t)sq * a.H + h) * a.splits + sp) * 16;
    a.part_o[pb * A_DH + tid] = num;
    if (tid == 0) {
      a.part_ml[pb * 2] = mstar;
      a.part_ml[pb * 2 + 1] = den;
    }
  }
}

void launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.M == 1) {
    // the row kernel, then (more than one split) the merge; ctx_stride is
    // a multiple of 64 (the engine aligns it, la_attention checks it)
    if (a.H * a.nseq < 1024)
      hipLaunchKernelGGL((k_attn_row<4, true>), dim3(a.H, a.splits, a.nseq), dim3(4 * 64), 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_row<4, false>), dim3(a.H, a.splits, a.nseq), dim3(4 * 64), 0, s, a);
    if (a.splits > 1) hipLaunchKernelGGL(k_attn_merge, dim3(1, a.H, a.nseq), dim3(256), 0, s, a);
    return;
  }
  if (attn_bf16_tiled(a.M, a.ctx_stride, a.H, a.nseq)) {
    hipLaunchKernelGGL(k_attn_tile, dim3(a.H, (a.M + 15) / 16, a.nseq), dim3(AT_NW * 64), 0, s, a);
    return;
  }
  // 2 key halves and a 2-chunk ring per workgroup; up to 32 rows one row
  // pair (72 KiB of LDS, two workgroups per CU), 33-64 rows two row pairs
  // (80 KiB), 65-128 rows row groups of 32 (measured at 121 rows and 0-1000
  // committed tokens: 1-4 us per layer faster than one 128-row workgroup per
  // head; at 57 rows, 64 heads and 2100 tokens one 64-row group is 3.7 us
  // faster than two of 32); above 128 rows one workgroup of 8 row pairs per
  // head.  attn_row_groups and attn_waves mirror this choice.
  if (a.M <= 32)
    launch_attn_inst<1, 2, 2>(a, s);
  else if (a.M <= 64)
    launch_attn_inst<2, 2, 2>(a, s);
  else if (a.M <= 128)
    launch_attn_inst<1, 2, 2>(a, s);
  else
    launch_attn_inst<8, 1, 2>(a, s);
  if (a.splits > 1)
    hipLaunchKernelGGL(k_attn_merge, dim3((a.M + 7) / 8, a.H, a.nseq), dim3(256), 0, s, a);
}

// ---------------------------------------------------------------------------
// fp32 kernel (small models, head_dim <= 256): one wave per (row, head),
// scores for every key in LDS, exact softmax.

__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
  extern __shared__ float sc[];
  const int t = blockIdx.x, h = blockIdx.y, sq = blockIdx.z, tid = threadIdx.x;
  const int L = a.st ? a.st[sq].L : a.L_host;
  const int M = a.M, dh = a.dh;
  const int kvh = (h * a.Hkv) / a.H;
  const int ctx = L + M;
  const int tg = sq * a.rps + t;  // row in q and out
  const float* q = (const float*)a.q + (size_t)tg * a.H * dh + (size_t)h * dh;
  const float* kc = (const float*)a.k_cache + sq * a.kv_seq + (size_t)kvh * a.ctx_stride * dh;
  const float* vc = (const float*)a.vt_cache + sq * a.kv_seq + (size_t)kvh * dh * a.ctx_stride;
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
  float* out = (float*)a.out + (size_t)tg * a.H * dh + (size_t)h * dh;
  for (int i = tid; i < dh; i += 64) {
    const float* v = vc + (size_t)i * a.ctx_stride;
    float acc = 0.f;
    for (int j = 0; j < ctx; j++) acc = fmaf(sc[j], v[j], acc);
    out[i] = acc / z;
  }
}

void launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_attn_f32, dim3(a.M, a.H, a.nseq), dim3(64), sizeof(float) * a.ctx_stride, s,
                     a);
}

}  // namespace la
