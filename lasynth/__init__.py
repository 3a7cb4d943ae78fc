"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and lays them out; it holds none of the
decoding method's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP
library (``lookahead_decoding_la_amd``) take their inputs from here, so that
each can be checked against the other on identical data.

The workloads follow the model sizes and lookahead settings the paper "Break
the Sequential Dependency of LLM Inference Using Lookahead Decoding" reports
as near-optimal (Key points, "Tuning knobs": 7B W=15 N=5, 13B W=10 N=5,
34B W=7 N=5, with G = W).  The paper's benchmarks (MT-Bench, HumanEval,
ClassEval) and LLaMA-2 weights are not available, so every input here is a
seeded stand-in: random-init weights N(0, 0.02) and synthetic prompts with
repeated spans (a Zipf(1.1) token distribution, as a stand-in for natural
text and code).

Randomness: every array comes from ``numpy.random.SeedSequence(seed,
spawn_key=...)`` with a fixed spawn key, so results do not depend on thread
count or call order.  Spawn keys: (0, tensor, chunk) weights; (1,) prompt;
(2,) initial lookahead window; (3, i) kernel-only attention inputs.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, replace

import numpy as np

# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    W: int
    N: int
    G: int
    prompt_len: int
    gen_tokens: int
    dtype: str  # "f32" or "bf16": weights, activations and KV cache
    prompt_kind: str  # "motif" (tiny) or "zipf"
    span_len: int = 16
    n_spans: int = 4
    span_repeats: int = 2
    rope_theta: float = 10000.0
    rms_eps: float = 1e-5

    @property
    def T(self) -> int:
        """Rows of one lookahead step: current token + window + candidates."""
        return 1 + (self.W + self.G) * (self.N - 1)

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


CONFIGS = {
    # 2 layers, d 128, 4 heads x 32, SwiGLU 344, vocab 512; W5 N3 G5; fp32.
    "tiny": ModelConfig("tiny", 2, 128, 4, 4, 32, 344, 512, 5, 3, 5,
                        prompt_len=32, gen_tokens=64, dtype="f32",
                        prompt_kind="motif"),
    # LLaMA-2-7B shape; W15 N5 G15 -> 121 rows per step.
    "7b": ModelConfig("7b", 32, 4096, 32, 32, 128, 11008, 32000, 15, 5, 15,
                      prompt_len=512, gen_tokens=256, dtype="bf16",
                      prompt_kind="zipf", span_len=16, n_spans=4,
                      span_repeats=2),
    # LLaMA-2-13B shape; W10 N5 G10 -> 81 rows per step.
    "13b": ModelConfig("13b", 40, 5120, 40, 40, 128, 13824, 32000, 10, 5, 10,
                       prompt_len=1024, gen_tokens=256, dtype="bf16",
                       prompt_kind="zipf", span_len=16, n_spans=8,
                       span_repeats=2),
    # 34B shape with grouped-query attention (64 q / 8 kv heads); W7 N5 G7.
    "34b": ModelConfig("34b", 48, 8192, 64, 8, 128, 22016, 32000, 7, 5, 7,
                       prompt_len=2048, gen_tokens=256, dtype="bf16",
                       prompt_kind="zipf", span_len=32, n_spans=4,
                       span_repeats=4),
}

# Kernel-only masked attention workload: 32 heads x 128, prefix 1024,
# W15 N5 G15 -> 121 query rows.
ATTN = dict(n_heads=32, n_kv_heads=32, head_dim=128, prefix=1024,
            W=15, N=5, G=15, vocab=32000)


def get_config(config_name: str, **overrides) -> ModelConfig:
    cfg = CONFIGS[config_name]
    return cfg.with_(**overrides) if overrides else cfg


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

_CHUNK = 1 << 24  # elements per independently seeded chunk


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16, nearest-even, returning the uint16 bit patterns.

    Inputs here are finite normal draws; NaN handling is not needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32)


def _normal_chunked(seed, tidx, n, std, bf16, pool):
    """n draws of N(0, std^2) in independently seeded chunks (parallel)."""
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)

    def work(ci):
        lo = ci * _CHUNK
        hi = min(n, lo + _CHUNK)
        x = _rng(seed, 0, tidx, ci).standard_normal(hi - lo, dtype=np.float32)
        x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x) if bf16 else x

    list(pool.map(work, range((n + _CHUNK - 1) // _CHUNK)))
    return out


def weight_shapes(cfg: ModelConfig):
    """(name, shape) of every tensor, in the fixed order both sides use.

    Matrices are row-major [out_features][in_features].
    """
    d, hd = cfg.d_model, cfg.head_dim
    shapes = [("tok_emb", (cfg.vocab, d)), ("final_norm", (d,)),
              ("lm_head", (cfg.vocab, d))]
    for l in range(cfg.n_layers):
        shapes += [
            (f"l{l}.attn_norm", (d,)),
            (f"l{l}.wq", (cfg.n_heads * hd, d)),
            (f"l{l}.wk", (cfg.n_kv_heads * hd, d)),
            (f"l{l}.wv", (cfg.n_kv_heads * hd, d)),
            (f"l{l}.wo", (d, cfg.n_heads * hd)),
            (f"l{l}.ffn_norm", (d,)),
            (f"l{l}.w_gate", (cfg.d_ffn, d)),
            (f"l{l}.w_up", (cfg.d_ffn, d)),
            (f"l{l}.w_down", (d, cfg.d_ffn)),
        ]
    return shapes


def make_weights(cfg: ModelConfig, seed: int = 0, threads: int | None = None):
    """Random-init weights: N(0, 0.02) everywhere, norm weights 1.0.

    Returns a list of numpy arrays in ``weight_shapes`` order: float32 for
    ``dtype == "f32"``; for ``"bf16"`` uint16 bit patterns of the fp32 draws
    rounded to bfloat16 (nearest-even), so that both sides see the same
    values exactly.
    """
    bf16 = cfg.dtype == "bf16"
    threads = threads or min(16, os.cpu_count() or 1)
    out = []
    with _cf.ThreadPoolExecutor(threads) as pool:
        for ti, (name, shape) in enumerate(weight_shapes(cfg)):
            n = int(np.prod(shape))
            if name.endswith("norm"):
                one = np.ones(n, np.float32)
                a = f32_to_bf16_bits(one) if bf16 else one
            else:
                a = _normal_chunked(seed, ti, n, 0.02, bf16, pool)
            out.append(a.reshape(shape))
    return out


def _tensor_seed(seed: int, tidx: int) -> int:
    return int(np.random.SeedSequence(seed, spawn_key=(0, tidx, 1 << 20))
               .generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def make_weights_device(cfg: ModelConfig, seed: int = 0, device="cuda"):
    """Random-init weights drawn on the GPU with torch's seeded generator
    (for the multi-billion-parameter workloads, where host generation is too
    slow).  Same recipe as make_weights -- N(0, 0.02) in fp32, rounded to
    bf16 (torch's float->bfloat16 conversion rounds to nearest even), norm
    weights 1.0 -- but a different random stream: tensor i is drawn from its
    own generator seeded from SeedSequence(seed, spawn_key=(0, i, 2**20)).
    Returns torch tensors (bfloat16 or float32) in weight_shapes order; the
    oracle side takes host copies of these same tensors (host_bits)."""
    import torch
    out = []
    for ti, (name, shape) in enumerate(weight_shapes(cfg)):
        if name.endswith("norm"):
            t = torch.ones(shape, dtype=torch.float32, device=device)
        else:
            g = torch.Generator(device=device)
            g.manual_seed(_tensor_seed(seed, ti))
            t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
            t.mul_(0.02)
        out.append(t.to(torch.bfloat16) if cfg.dtype == "bf16" else t)
    return out


def host_bits(tensors):
    """Host numpy copies of device weight tensors: bfloat16 as uint16 bit
    patterns, float32 as float32 (the layout make_weights returns)."""
    import torch
    out = []
    for t in tensors:
        if t.dtype == torch.bfloat16:
            out.append(t.view(torch.int16).cpu().numpy().view(np.uint16))
        else:
            out.append(t.cpu().numpy())
    return out


# ----------------------------------------------------------------------------
# prompts and windows
# ----------------------------------------------------------------------------


def _zipf_tokens(rng, n, vocab, a=1.1):
    """n tokens: Zipf(a) ranks truncated to [1, vocab] by rejection, id = rank-1."""
    got = np.empty(0, dtype=np.int64)
    while got.size < n:
        z = rng.zipf(a, size=2 * (n - got.size) + 16)
        got = np.concatenate([got, z[z <= vocab]])
    return (got[:n] - 1).astype(np.int32)


def make_prompt(cfg: ModelConfig, seed: int = 0) -> np.ndarray:
    rng = _rng(seed, 1)
    P, V = cfg.prompt_len, cfg.vocab
    if cfg.prompt_kind == "motif":
        # layout R4 M8 R2 M8 R2 M8 (R = fresh uniform tokens, M = one motif),
        # scaled to the prompt length when it is not 32.
        motif = rng.integers(0, V, size=8, dtype=np.int64)
        parts = []
        for r in (4, 2, 2):
            parts.append(rng.integers(0, V, size=r, dtype=np.int64))
            parts.append(motif)
        p = np.concatenate(parts)
        if P > p.size:
            p = np.concatenate([p, rng.integers(0, V, size=P - p.size)])
        return p[:P].astype(np.int32)
    # Zipf(1.1) background with n_spans distinct spans, each placed
    # span_repeats times at distinct span-aligned slots.
    p = _zipf_tokens(rng, P, V)
    S, n_sp, rep = cfg.span_len, cfg.n_spans, cfg.span_repeats
    n_slots = P // S
    need = n_sp * rep
    if need > n_slots:
        raise ValueError("prompt too short for its repeated spans")
    slots = rng.permutation(n_slots)[:need]
    for s in range(n_sp):
        span = _zipf_tokens(rng, S, V)
        for r in range(rep):
            o = int(slots[s * rep + r]) * S
            p[o:o + S] = span
    return p.astype(np.int32)


def make_init_window(cfg: ModelConfig, prompt: np.ndarray,
                     seed: int = 0) -> np.ndarray:
    """Initial lookahead window, (N-1) levels x W columns, row = level.

    Each entry is a prompt token at a uniformly drawn index.
    """
    rng = _rng(seed, 2)
    n = (cfg.N - 1) * cfg.W
    idx = rng.integers(0, len(prompt), size=n)
    return np.asarray(prompt, np.int32)[idx].reshape(cfg.N - 1, cfg.W).copy()


# ----------------------------------------------------------------------------
# kernel-only attention workload
# ----------------------------------------------------------------------------


def make_attn_inputs(seed: int = 0, n_heads=None, n_kv_heads=None,
                     head_dim=None, prefix=None, W=None, N=None, G=None):
    """Q [T][H][dh], K and V [Hkv][prefix+T][dh], all N(0,1) rounded to bf16
    (uint16 bit patterns); candidate tokens [G][N-1] uniform over the vocab
    (they do not enter attention).
    """
    H = n_heads or ATTN["n_heads"]
    Hkv = n_kv_heads or (H if n_heads else ATTN["n_kv_heads"])
    dh = head_dim or ATTN["head_dim"]
    L = ATTN["prefix"] if prefix is None else prefix
    W = ATTN["W"] if W is None else W
    N = ATTN["N"] if N is None else N
    G = ATTN["G"] if G is None else G
    T = 1 + (W + G) * (N - 1)

    def draw(i, shape):
        x = _rng(seed, 3, i).standard_normal(int(np.prod(shape)),
                                              dtype=np.float32)
        return f32_to_bf16_bits(x).reshape(shape)

    q = draw(0, (T, H, dh))
    k = draw(1, (Hkv, L + T, dh))
    v = draw(2, (Hkv, L + T, dh))
    cands = _rng(seed, 3, 3).integers(0, ATTN["vocab"], size=(G, N - 1),
                                      dtype=np.int64).astype(np.int32)
    return dict(q=q, k=k, v=v, cands=cands, prefix=L, W=W, N=N, G=G, T=T,
                n_heads=H, n_kv_heads=Hkv, head_dim=dh)
