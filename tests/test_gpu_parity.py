"""HIP decoder vs CPU oracle, in lockstep, through the C ABI (GPU only).

Tolerances (floating point decides integers only through argmax, compared
with the near-tie rule of tests/lockstep.py):
  - fp32 models: logits within 1e-4, argmax mismatches only where the
    oracle's top-2 margin is <= 2e-4;
  - bf16 models: logits within 2e-2, argmax mismatches only where the
    oracle's top-2 margin is <= 0.05;
  - tokens, accepted lengths, window and pool bit-exact (after adoption of
    excused near-ties).
"""
import numpy as np
import pytest

import lasynth
import oracle
from lockstep import Lockstep, log

pytestmark = pytest.mark.gpu

FP32 = [
    lasynth.get_config("tiny"),
    lasynth.get_config("tiny", name="tiny_n2", N=2),
    lasynth.get_config("tiny", name="tiny_verify_only", W=0, G=3),
    lasynth.get_config("tiny", name="tiny_lookahead_only", W=4, G=0),
    lasynth.get_config("tiny", name="tiny_gqa_n5", n_heads=4, n_kv_heads=2, N=5, W=3, G=4),
    lasynth.get_config("tiny", name="tiny_plain", W=0, G=0),
    # the largest step the kernels take: 1 + (26 + 25) * 5 = 256 rows
    lasynth.get_config("tiny", name="tiny_t256", N=6, W=26, G=25, gen_tokens=48),
]


@pytest.mark.parametrize("cfg", FP32, ids=lambda c: c.name)
def test_fp32_lockstep(cfg):
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p) if cfg.W else None
    log(f"[fp32 lockstep] {cfg.name} T={cfg.T}")
    ls = Lockstep(cfg, w, 512, logit_tol=1e-4, tie_margin=2e-4)
    toks = ls.run(p, win, M=cfg.gen_tokens)
    ls.compare_kv(1e-4)
    log(f"  steps={len(ls.steps)} max|dlogit|={ls.max_diff:.2e} ties={ls.ties}")
    # and the output is plain greedy decoding, up to the first step that
    # adopted an excused decision (the oracle's greedy run never adopts)
    M = cfg.gen_tokens
    n = min(ls.tokens_before_first_excuse(toks), M)
    assert toks[:n] == oracle.Oracle(cfg, w, 512).greedy(p, M)[:n]
    log(f"  {n} of {M} tokens compared with plain greedy decoding")


BF16 = [
    # 121 rows per step (W15 N5 G15) as in the 7B workload, narrow model
    lasynth.get_config("7b", name="bf16_w15", n_layers=3, d_model=512, n_heads=4,
                       n_kv_heads=4, d_ffn=1408, vocab=2048, prompt_len=64,
                       span_len=8, n_spans=2),
    # grouped KV heads, 57 rows per step (W7 N5 G7, the 34B setting)
    lasynth.get_config("34b", name="bf16_gqa_w7", n_layers=2, d_model=1024, n_heads=8,
                       n_kv_heads=2, d_ffn=2816, vocab=4096, prompt_len=96,
                       span_len=8, n_spans=2, span_repeats=3),
    # ragged: 81 rows (W10 N5 G10), 1 layer, prompt longer than one chunk
    lasynth.get_config("13b", name="bf16_w10_long", n_layers=1, d_model=256, n_heads=2,
                       n_kv_heads=2, d_ffn=704, vocab=1024, prompt_len=300,
                       span_len=16, n_spans=4),
    # 161 rows (W20 N5 G20): the attention variant for more than 128 rows,
    # in the step and in 192-row prefill chunks
    lasynth.get_config("7b", name="bf16_w20_t161", n_layers=2, d_model=256, n_heads=2,
                       n_kv_heads=2, d_ffn=704, vocab=1024, prompt_len=300, W=20, G=20,
                       span_len=8, n_spans=2),
    # the largest step: 256 rows (W26 N6 G25); 16-token-tile GEMMs, a
    # 300-token prompt prefilled as a full 256-row chunk plus a ragged 44
    lasynth.get_config("7b", name="bf16_max_t256", n_layers=1, d_model=256, n_heads=2,
                       n_kv_heads=2, d_ffn=704, vocab=1024, prompt_len=300, N=6, W=26, G=25,
                       span_len=8, n_spans=2),
    # plain one-token decode
    lasynth.get_config("7b", name="bf16_plain", n_layers=2, d_model=512, n_heads=4,
                       n_kv_heads=4, d_ffn=1408, vocab=2048, prompt_len=64,
                       span_len=8, n_spans=2, W=0, G=0),
    # an 11-row block (W2 N3 G3): at most 12 rows, so the one-tile GEMMs
    # with their fused epilogues carry the lookahead step
    lasynth.get_config("7b", name="bf16_t11", n_layers=2, d_model=512, n_heads=4,
                       n_kv_heads=4, d_ffn=1408, vocab=2048, prompt_len=64,
                       span_len=8, n_spans=2, W=2, N=3, G=3),
    # a 12-token prompt: the prefill itself is a one-tile pass (causal rows)
    lasynth.get_config("7b", name="bf16_t11_short_prompt", n_layers=2, d_model=512, n_heads=4,
                       n_kv_heads=2, d_ffn=1408, vocab=2048, prompt_len=12,
                       span_len=4, n_spans=1, W=2, N=3, G=3),
    # a wide FFN (1056 gate/up tile pairs, as the 34B shape's 1376: dealt
    # over 256 twelve-wave workgroups) and a 16-way split of the down GEMM;
    # 57-row steps and plain decode
    lasynth.get_config("34b", name="bf16_wide_ffn_w7", n_layers=1, d_model=256, n_heads=2,
                       n_kv_heads=2, d_ffn=16896, vocab=1024, prompt_len=96,
                       span_len=8, n_spans=2),
    lasynth.get_config("34b", name="bf16_wide_ffn_plain", n_layers=1, d_model=256, n_heads=2,
                       n_kv_heads=2, d_ffn=16896, vocab=1024, prompt_len=96,
                       span_len=8, n_spans=2, W=0, G=0),
    # N = 2 (a window of one level, one-token candidates), 17 rows: the
    # register-ring GEMMs (two token tiles)
    lasynth.get_config("7b", name="bf16_n2_w8", n_layers=2, d_model=512, n_heads=4,
                       n_kv_heads=4, d_ffn=1408, vocab=2048, prompt_len=64,
                       span_len=8, n_spans=2, W=8, N=2, G=8),
    # a one-token prompt (a one-row causal prefill), then 9-row steps
    lasynth.get_config("7b", name="bf16_prompt1_n2", n_layers=2, d_model=512, n_heads=4,
                       n_kv_heads=4, d_ffn=1408, vocab=2048, prompt_len=1,
                       span_len=1, n_spans=0, W=4, N=2, G=4),
    # cache rows above 2048 keys (capacity LONG_CTX): the split attention for
    # the 128- and 44-row causal prefill chunks of a 300-token prompt and for
    # the 57-row steps
    lasynth.get_config("34b", name="bf16_long_ctx_w7", n_layers=1, d_model=256, n_heads=2,
                       n_kv_heads=2, d_ffn=704, vocab=1024, prompt_len=300,
                       span_len=16, n_spans=4),
]
LONG_CTX = {"bf16_long_ctx_w7": 2304}


@pytest.mark.parametrize("cfg", BF16, ids=lambda c: c.name)
def test_bf16_lockstep(cfg):
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p) if cfg.W else None
    log(f"[bf16 lockstep] {cfg.name} T={cfg.T}")
    ls = Lockstep(cfg, w, LONG_CTX.get(cfg.name, 1024), logit_tol=2e-2)
    ls.run(p, win, n_steps=10)
    ls.compare_kv(3e-2)
    log(f"  steps={len(ls.steps)} max|dlogit|={ls.max_diff:.2e} ties={ls.ties}")


def test_planted_candidate_accepted_on_gpu():
    cfg = BF16[0]
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p)
    ls = Lockstep(cfg, w, 512, logit_tol=2e-2)
    out = [ls.prefill(p, win)]
    greedy = oracle.Oracle(cfg, w, 512).greedy(p, 40)
    if ls.ties:
        pytest.skip("prefill token decided by a near-tie")
    for _ in range(4):
        n = len(out)
        tail = greedy[n:n + cfg.N - 1]
        ls.dev.debug_pool_insert(out[-1], tail)
        ls.orc.pool_insert(out[-1], tail)
        r = ls.step()
        if ls.ties:
            break
        assert r["accepted"] == cfg.N - 1
        assert r["tokens"] == greedy[n:n + cfg.N]
        out += r["tokens"]


@pytest.mark.parametrize("cfg", [FP32[0], BF16[0]], ids=lambda c: c.name)
def test_prompt_ngram_seeding(cfg):
    """Pool seeded with the prompt's n-grams (Key points, "Ablation"): the
    seeded pools agree bit-exactly, and the lockstep steps that follow
    (candidates now drawn from the prompt) agree as everywhere else."""
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p)
    tol = 1e-4 if cfg.dtype == "f32" else 2e-2
    ls = Lockstep(cfg, w, 512, logit_tol=tol, tie_margin=2e-4 if cfg.dtype == "f32" else 0.05)
    ls.prefill(p, win)
    ls.seed(p)
    for _ in range(8):
        ls.step()
    log(f"  {cfg.name} seeded: steps={len(ls.steps)} max|dlogit|={ls.max_diff:.2e} ties={ls.ties}")


@pytest.mark.parametrize("cfg", [FP32[0], BF16[0]], ids=lambda c: c.name)
def test_step_past_capacity_is_refused(cfg):
    """A step whose rows would not fit in max_ctx is refused with
    LA_ERR_OUT_OF_CAPACITY before anything is launched: the steps up to the
    limit agree with the oracle, and the refused step leaves the cache
    length, current token, window and pool as they were."""
    import lookahead_decoding_la_amd as la
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p)
    tol = 1e-4 if cfg.dtype == "f32" else 2e-2
    max_ctx = len(p) + cfg.T + 40
    ls = Lockstep(cfg, w, max_ctx, logit_tol=tol, tie_margin=2e-4 if cfg.dtype == "f32" else 0.05)
    ls.prefill(p, win)
    while ls.orc.kv_len + cfg.T <= max_ctx:
        ls.step()
    before = (ls.dev.debug_state(), ls.dev.debug_window(), ls.dev.debug_pool())
    for _ in range(2):
        with pytest.raises(la.LaError) as e:
            ls.dev.step()
        assert e.value.status == la.LA_ERR_OUT_OF_CAPACITY
    after = (ls.dev.debug_state(), ls.dev.debug_window(), ls.dev.debug_pool())
    assert before[0] == after[0] == (ls.orc.kv_len, ls.orc.current)
    assert np.array_equal(before[1], after[1])
    assert np.array_equal(before[2][0], after[2][0]) and np.array_equal(before[2][1], after[2][1])
    log(f"  {cfg.name}: {len(ls.steps)} steps before the capacity limit (kv {ls.orc.kv_len})")
