"""Batched lookahead steps on the GPU: B sequences forwarded together, each
compared in lockstep with an oracle of its own (GPU only).

A batched step is by definition B independent single-sequence steps (each
sequence attends to its own cache and block), so the oracle of a batch is B
ordinary oracles.  Sequences get different prompts, prompt lengths and
windows, so their committed lengths, candidates and accepted lengths drift
apart step by step.  Tolerances as in tests/test_gpu_parity.py.
"""
import pytest

import lasynth
import oracle
from lockstep import BatchLockstep, log

pytestmark = pytest.mark.gpu


def _inputs(cfg, B, lengths):
    prompts, wins = [], []
    for b in range(B):
        c = cfg.with_(prompt_len=lengths[b % len(lengths)])
        p = lasynth.make_prompt(c, seed=b)
        prompts.append(p)
        wins.append(lasynth.make_init_window(c, p, seed=b) if cfg.W else None)
    return prompts, wins


CASES = [
    # (config, batch, prompt lengths, steps)
    (lasynth.get_config("tiny", name="tiny_b3"), 3, [32, 45, 27], 12),
    (lasynth.get_config("tiny", name="tiny_gqa_b4", n_heads=4, n_kv_heads=2, N=4, W=4, G=4),
     4, [30, 33, 41, 26], 10),
    (lasynth.get_config("tiny", name="tiny_plain_b8", W=0, G=0), 8, [20, 29, 31, 40], 12),
    # 2 x 121 rows: the 7B step shape on a narrow model
    (lasynth.get_config("7b", name="bf16_w15_b2", n_layers=2, d_model=512, n_heads=4,
                        n_kv_heads=4, d_ffn=1408, vocab=2048, span_len=8, n_spans=2),
     2, [64, 100], 8),
    # 4 x 57 rows, grouped KV heads (W7 N5 G7)
    (lasynth.get_config("34b", name="bf16_gqa_w7_b4", n_layers=2, d_model=1024, n_heads=8,
                        n_kv_heads=2, d_ffn=2816, vocab=4096, span_len=8, n_spans=2),
     4, [96, 70, 130, 81], 8),
    # 16 plain one-token decodes
    (lasynth.get_config("7b", name="bf16_plain_b16", n_layers=2, d_model=512, n_heads=4,
                        n_kv_heads=4, d_ffn=1408, vocab=2048, span_len=8, n_spans=2,
                        W=0, G=0),
     16, [40, 64, 51], 8),
    # passes of at most 12 rows take the one-tile GEMMs, whose QKV epilogue
    # places each row's K/V in its own sequence's cache: 8 one-row
    # sequences, and 2 sequences of 5-row lookahead blocks (W1 N3 G1)
    (lasynth.get_config("7b", name="bf16_plain_b8_one_tile", n_layers=2, d_model=512, n_heads=4,
                        n_kv_heads=2, d_ffn=1408, vocab=2048, span_len=8, n_spans=2,
                        W=0, G=0),
     8, [40, 64, 51], 8),
    (lasynth.get_config("7b", name="bf16_t5_b2_one_tile", n_layers=2, d_model=512, n_heads=4,
                        n_kv_heads=4, d_ffn=1408, vocab=2048, span_len=8, n_spans=2,
                        W=1, N=3, G=1),
     2, [64, 45], 10),
    # one-token decodes over long prompts: up to 8 key splits per head and
    # their merge
    (lasynth.get_config("7b", name="bf16_plain_b2_long", n_layers=2, d_model=512, n_heads=4,
                        n_kv_heads=4, d_ffn=1408, vocab=2048, span_len=8, n_spans=2,
                        W=0, G=0),
     2, [600, 350], 8),
    # 8 sequences of 21-row blocks (W5 N3 G5), 16 heads: heads x tiles x
    # sequences fill 256 CUs, so the small blocks take the per-tile kernel
    (lasynth.get_config("7b", name="bf16_w5n3g5_b8", n_layers=2, d_model=1024, n_heads=16,
                        n_kv_heads=16, d_ffn=2816, vocab=4096, span_len=8, n_spans=2,
                        W=5, N=3, G=5),
     8, [40, 64, 51], 6),
    # 64 plain one-token decodes of 16 heads: 1024 (head, sequence) pairs
    # take the one-row attention kernel's shallow-prefetch form
    (lasynth.get_config("7b", name="bf16_plain_b64_h16", n_layers=2, d_model=1024, n_heads=16,
                        n_kv_heads=16, d_ffn=2816, vocab=4096, span_len=8, n_spans=2,
                        W=0, G=0),
     64, [40, 64, 51, 100], 4),
    # 40 plain one-token decodes of 8 heads (320 sequence heads): the most
    # sequences one context takes at one row each below the row cap
    (lasynth.get_config("7b", name="bf16_plain_b40", n_layers=2, d_model=1024, n_heads=8,
                        n_kv_heads=8, d_ffn=2816, vocab=4096, span_len=8, n_spans=2,
                        W=0, G=0),
     40, [40, 64, 51], 6),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_batch_lockstep(case):
    cfg, B, lengths, n_steps = case
    f32 = cfg.dtype == "f32"
    w = lasynth.make_weights(cfg)
    prompts, wins = _inputs(cfg, B, lengths)
    log(f"[batch lockstep] {cfg.name} B={B} T={cfg.T} rows={B * cfg.T}")
    ls = BatchLockstep(cfg, w, 1024, B, logit_tol=1e-4 if f32 else 2e-2,
                       tie_margin=2e-4 if f32 else 0.05)
    ls.prefill(prompts, wins)
    for _ in range(n_steps):
        ls.step()
    ls.compare_kv(1e-4 if f32 else 3e-2)
    acc = [sum(s[b]["n_emitted"] for s in ls.steps) for b in range(B)]
    log(f"  tokens per sequence {acc}, max|dlogit|={ls.max_diff:.2e} ties={ls.ties}")


def test_batch_sequence_restarts_alone():
    """Prefilling one sequence again (a new request in its slot) resets only
    that sequence: the others keep decoding as before."""
    cfg = lasynth.get_config("tiny", name="tiny_b3")
    B = 3
    w = lasynth.make_weights(cfg)
    prompts, wins = _inputs(cfg, B, [32, 45, 27])
    ls = BatchLockstep(cfg, w, 1024, B, logit_tol=1e-4, tie_margin=2e-4)
    ls.prefill(prompts, wins)
    for _ in range(4):
        ls.step()
    c2 = cfg.with_(prompt_len=38)
    p2 = lasynth.make_prompt(c2, seed=7)
    w2 = lasynth.make_init_window(c2, p2, seed=7)
    ls.orcs[1] = oracle.Oracle(cfg, w, 1024)
    ls.prefill_one(1, p2, w2)
    for _ in range(6):
        ls.step()
    log(f"  restarted sequence 1 at step 4: max|dlogit|={ls.max_diff:.2e} ties={ls.ties}")


def test_batch_capacity_refuses_every_sequence():
    """When any sequence lacks room for one more block, the whole batched
    step is refused and no sequence changes."""
    import lookahead_decoding_la_amd as la
    cfg = lasynth.get_config("tiny", name="tiny_b2")
    w = lasynth.make_weights(cfg)
    prompts, wins = _inputs(cfg, 2, [32, 120])
    max_ctx = 120 + cfg.T + 12
    ls = BatchLockstep(cfg, w, max_ctx, 2, logit_tol=1e-4, tie_margin=2e-4)
    ls.prefill(prompts, wins)
    while max(o.kv_len for o in ls.orcs) + cfg.T <= max_ctx:
        ls.step()
    before = ls.dev.debug_state()
    with pytest.raises(la.LaError) as e:
        ls.dev.step()
    assert e.value.status == la.LA_ERR_OUT_OF_CAPACITY
    assert ls.dev.debug_state() == before == [(o.kv_len, o.current) for o in ls.orcs]
    log(f"  refused after {len(ls.steps)} steps, states {before}")
