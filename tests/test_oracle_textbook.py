"""Pin the oracle's transformer arithmetic to an independent textbook decoder.

The textbook decoder below is written with torch float64 library routines
(embedding lookup, complex-number rotary embedding, scaled_dot_product_attention
with a causal mask, SiLU) and shares nothing with the oracle's C loops.  A
causal forward over a sequence must give the same logits for every row.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import lasynth
import oracle


def _w64(cfg, a):
    a = np.asarray(a)
    if cfg.dtype == "bf16":
        a = lasynth.bf16_bits_to_f32(a)
    return torch.from_numpy(np.asarray(a, np.float64))


def _bf16(x):
    """bfloat16 storage through torch's own conversion (float64 -> float32 ->
    bfloat16, round to nearest even), widened back to float64."""
    return x.to(torch.bfloat16).to(torch.float64)


def textbook_logits(cfg, weights, tokens, storage="exact"):
    """Causal logits of every row.  storage="bf16": the seven activations a
    bf16 datapath stores are rounded with torch's bfloat16 conversion (the
    normalized block inputs as bf16(x * w) with 1/rms applied to the
    products, q/k after the rotary embedding and v, the attention
    probabilities entering the value sum, the attention output, the SwiGLU
    output and the LM head's normalized input); attention is then written
    out (softmax with the rounded probabilities) instead of SDPA."""
    bf = storage == "bf16"
    names = [n for n, _ in lasynth.weight_shapes(cfg)]
    W = {n: _w64(cfg, a) for n, a in zip(names, weights)}
    T = len(tokens)
    H, Hkv, dh = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim

    def norm(x, w):
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + cfg.rms_eps) * w

    pos = torch.arange(T, dtype=torch.float64)
    inv = cfg.rope_theta ** (-(torch.arange(0, dh, 2, dtype=torch.float64) / dh))
    rot = torch.polar(torch.ones(T, dh // 2, dtype=torch.float64),
                      pos[:, None] * inv[None, :])  # [T][dh/2] complex

    def rope(x):  # x [T][heads][dh], adjacent pairs as complex numbers
        xc = torch.view_as_complex(x.reshape(T, x.shape[1], dh // 2, 2).contiguous())
        return torch.view_as_real(xc * rot[:, None, :]).reshape(x.shape)

    def proj(x, wn, *mats):
        """x's RMSNorm (weights wn) times each matrix; bf16 storage holds
        bf16(x * wn) and scales the products by 1/rms."""
        if not bf:
            n = norm(x, wn)
            return [n @ m.T for m in mats]
        n = _bf16(x * wn)
        s = torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + cfg.rms_eps)
        return [(n @ m.T) * s for m in mats]

    keep = _bf16 if bf else (lambda t: t)
    causal = torch.ones(T, T, dtype=torch.bool).tril()
    x = F.embedding(torch.as_tensor(tokens, dtype=torch.long), W["tok_emb"])
    for l in range(cfg.n_layers):
        q, k, v = proj(x, W[f"l{l}.attn_norm"], W[f"l{l}.wq"], W[f"l{l}.wk"], W[f"l{l}.wv"])
        q = keep(rope(q.reshape(T, H, dh)))
        k = keep(rope(k.reshape(T, Hkv, dh)))
        v = keep(v.reshape(T, Hkv, dh))
        k = k.repeat_interleave(H // Hkv, dim=1)
        v = v.repeat_interleave(H // Hkv, dim=1)
        if not bf:
            a = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1),
                                               v.transpose(0, 1), is_causal=True)
        else:
            sc = (q.transpose(0, 1) @ k.permute(1, 2, 0)) / dh ** 0.5  # [H][T][T]
            sc = sc.masked_fill(~causal, float("-inf"))
            p = torch.exp(sc - sc.amax(-1, keepdim=True))
            a = keep((keep(p) @ v.transpose(0, 1)) / p.sum(-1, keepdim=True))
        x = x + a.transpose(0, 1).reshape(T, H * dh) @ W[f"l{l}.wo"].T
        g, u = proj(x, W[f"l{l}.ffn_norm"], W[f"l{l}.w_gate"], W[f"l{l}.w_up"])
        x = x + keep(F.silu(g) * u) @ W[f"l{l}.w_down"].T
    return (keep(norm(x, W["final_norm"])) @ W["lm_head"].T).numpy()


SMALL = [
    lasynth.get_config("tiny"),
    # grouped-query attention, odd FFN width
    lasynth.get_config("tiny", name="gqa", d_model=64, n_heads=4, n_kv_heads=2,
                       head_dim=16, d_ffn=96, vocab=300, n_layers=2),
    # bfloat16 weights, 3 layers
    lasynth.get_config("tiny", name="bf16", dtype="bf16", n_layers=3, d_model=96,
                       n_heads=3, n_kv_heads=1, head_dim=32, d_ffn=200, vocab=257),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_causal_logits_match_textbook(cfg):
    w = lasynth.make_weights(cfg, seed=3)
    rng = np.random.default_rng(5)
    toks = rng.integers(0, cfg.vocab, size=40).astype(np.int32)
    o = oracle.Oracle(cfg, w, 64)
    _, lg = o.extend(toks, logits=True)
    ref = textbook_logits(cfg, w, toks)
    assert np.max(np.abs(lg - ref)) < 1e-9


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_bf16_storage_logits_match_textbook(cfg):
    """The oracle's bf16 storage mode against the textbook decoder rounding
    the same seven activations with torch's bfloat16 conversion."""
    w = lasynth.make_weights(cfg, seed=3)
    toks = np.random.default_rng(5).integers(0, cfg.vocab, size=40).astype(np.int32)
    o = oracle.Oracle(cfg, w, 64, storage="bf16")
    _, lg = o.extend(toks, logits=True)
    ref = textbook_logits(cfg, w, toks, storage="bf16")
    assert np.max(np.abs(lg - ref)) < 1e-9
    # and the storage changes the logits (by rounding-sized amounts)
    exact = textbook_logits(cfg, w, toks)
    d = np.max(np.abs(lg - exact))
    assert 1e-5 < d < 0.1, d


def test_chunked_prefill_is_bit_identical(tiny):
    cfg, w, p, _ = tiny
    a = oracle.Oracle(cfg, w, 128)
    _, lg_a = a.extend(p, logits=True)
    b = oracle.Oracle(cfg, w, 128)
    _, l1 = b.extend(p[:13], logits=True)
    _, l2 = b.extend(p[13:], logits=True)
    assert np.array_equal(lg_a, np.concatenate([l1, l2]))
    for layer in range(cfg.n_layers):
        ka, va = a.kv(layer, 0, len(p))
        kb, vb = b.kv(layer, 0, len(p))
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_thread_count_does_not_change_results(tiny):
    cfg, w, p, win = tiny
    prev = oracle.max_threads()
    oracle.set_threads(1)
    try:
        a = oracle.Oracle(cfg, w, 128)
        a.prefill(p, win)
        ra, la = a.step(logits=True)
    finally:
        oracle.set_threads(prev)
    b = oracle.Oracle(cfg, w, 128)
    b.prefill(p, win)
    rb, lb = b.step(logits=True)
    assert ra == rb
    assert np.array_equal(la, lb, equal_nan=True)
