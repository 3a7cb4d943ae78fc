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


def textbook_logits(cfg, weights, tokens):
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

    x = F.embedding(torch.as_tensor(tokens, dtype=torch.long), W["tok_emb"])
    for l in range(cfg.n_layers):
        n = norm(x, W[f"l{l}.attn_norm"])
        q = rope((n @ W[f"l{l}.wq"].T).reshape(T, H, dh))
        k = rope((n @ W[f"l{l}.wk"].T).reshape(T, Hkv, dh))
        v = (n @ W[f"l{l}.wv"].T).reshape(T, Hkv, dh)
        k = k.repeat_interleave(H // Hkv, dim=1)
        v = v.repeat_interleave(H // Hkv, dim=1)
        a = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1),
                                           v.transpose(0, 1), is_causal=True)
        x = x + a.transpose(0, 1).reshape(T, H * dh) @ W[f"l{l}.wo"].T
        n = norm(x, W[f"l{l}.ffn_norm"])
        h = F.silu(n @ W[f"l{l}.w_gate"].T) * (n @ W[f"l{l}.w_up"].T)
        x = x + h @ W[f"l{l}.w_down"].T
    return (norm(x, W["final_norm"]) @ W["lm_head"].T).numpy()


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
