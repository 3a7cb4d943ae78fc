"""Pin the oracle's bf16 storage mode (the model of a bf16 datapath, where
seven activations per layer are stored as bfloat16; the pages fix no number
format, so this precision is a reading).

- The rounding itself equals torch's bfloat16 conversion of the same
  float64 values (float64 -> float32 -> bfloat16, nearest even), including
  exact ties at both steps.
- The method's exactness holds in this mode as in the exact one: lookahead
  output equals plain greedy decoding, and every block row equals a causal
  re-run of the sequence the mask implies, bit for bit.
- Committed K/V values are bfloat16 values.
(The model-level rounding points are pinned against the textbook decoder in
test_oracle_textbook.py.)
"""
import numpy as np
import pytest
import torch

import lasynth
import oracle


def test_round_bf16_equals_torch_conversion():
    rng = np.random.default_rng(7)
    vals = rng.normal(size=4000) * 10.0 ** rng.uniform(-8, 8, 4000)
    # exact bf16 midpoints (fp32 words ending in 0x8000), and fp64 values a
    # hair either side of them and of fp32 midpoints
    mids = (rng.integers(0x3000, 0x5000, 2000, dtype=np.uint32) << 16) | 0x8000
    m = mids.view(np.float32).astype(np.float64)
    ulp32 = np.spacing(m.astype(np.float32)).astype(np.float64)
    vals = np.concatenate([vals, m, -m, m + ulp32 / 4, m - ulp32 / 4, m + ulp32 / 2,
                           m - ulp32 / 2, m * (1 + 2.0 ** -40), [0.0, -0.0, 1.0, 3.0]])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_bf16(v) for v in vals])
    assert np.array_equal(got, ref)


CFGS = [
    lasynth.get_config("tiny"),
    lasynth.get_config("tiny", name="bf16_gqa", dtype="bf16", d_model=64, n_heads=4,
                       n_kv_heads=2, head_dim=16, d_ffn=96, vocab=300, W=4, N=4, G=3),
]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_bf16_storage_lookahead_equals_greedy(cfg):
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p)
    M = 48
    toks, steps = oracle.Oracle(cfg, w, 256, storage="bf16").generate(p, win, M,
                                                                       seed_prompt=True)
    assert toks == oracle.Oracle(cfg, w, 256, storage="bf16").greedy(p, M)
    assert sum(s["n_emitted"] for s in steps) > len(steps)  # something was accepted


def test_bf16_storage_block_rows_equal_causal_rerun(tiny):
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 256, storage="bf16")
    gen = [o.prefill(p, win)]
    rng = np.random.default_rng(2)
    for step in range(3):
        o.pool_insert(o.current, rng.integers(0, cfg.vocab, cfg.N - 1))
        tok, valid, _ = o.block_tokens()
        committed = (list(p) + gen)[:o.kv_len]
        lg = o.forward_block(tok, valid, keep=True)
        for r in np.nonzero(valid)[0]:
            vis = sorted((s for s in range(cfg.T) if oracle.visible(cfg, r, s)),
                         key=lambda s: oracle.row_pos(cfg, s))
            ref = oracle.Oracle(cfg, w, 256, storage="bf16")
            _, rl = ref.extend(committed + [int(tok[s]) for s in vis], logits=True)
            assert np.array_equal(rl[-1], lg[r]), (step, r)
        gen += o.commit()["tokens"]


def test_bf16_storage_kv_holds_bf16_values(tiny):
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 256, storage="bf16")
    o.prefill(p, win)
    o.step()
    e = oracle.Oracle(cfg, w, 256)
    e.prefill(p, win)
    e.step()
    for layer in range(cfg.n_layers):
        k, v = o.kv(layer, 0, o.kv_len)
        for a in (k, v):
            f = a.astype(np.float32)
            assert np.array_equal(f.astype(np.float64), a)
            assert not np.any(f.view(np.uint32) & 0xFFFF)
        ke, _ = e.kv(layer, 0, e.kv_len)
        assert not np.array_equal(k, ke)
