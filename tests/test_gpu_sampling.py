"""Sampled decoding on the GPU against the oracle (GPU only).

- The draw kernel on its own (la_sample): GPU draws equal the oracle's draws
  from the same fp32 logits with the same position-keyed uniforms, except
  where the oracle's draw sits within 1e-5 of a boundary (the two sides sum
  the weights in different orders, fp32 against fp64); and the drawn
  frequencies pass a chi-square test against the definition's
  probabilities.
- Whole steps in lockstep with the oracle (tests/lockstep.py) with
  sampling on, for fp32 and bf16 models, and in a batch that mixes greedy
  and sampled sequences.
- A property at any size: sampled lookahead decoding on the GPU emits the
  tokens of sampled plain decoding on the GPU with the same seed, up to a
  first divergence that must sit at a draw within the tolerance of a
  boundary.
"""
import math

import numpy as np
import pytest
import torch

import lasynth
import lookahead_decoding_la_amd as la
import oracle
from helpers import definition_probs
from lockstep import BatchLockstep, Lockstep, draw_tol, log

pytestmark = pytest.mark.gpu

PARAMS = [(1.0, 0, 1.0, 7), (0.7, 0, 0.9, 8), (1.3, 40, 1.0, 9), (0.5, 5, 0.8, 10),
          (2.0, 0, 0.5, 11),
          (1.0, 64, 0.7, 12),   # largest top-k drawn from the sorted kept tokens
          (0.9, 65, 0.95, 13)]  # smallest top-k on the whole-vocabulary searches


@pytest.mark.parametrize("T,k,p,seed", PARAMS)
def test_draw_kernel_matches_oracle(T, k, p, seed):
    rng = np.random.default_rng(seed)
    rows, V = 96, 32000
    lg = rng.normal(0, 2, (rows, V)).astype(np.float32)
    lg[5, :200] = lg[5, 0]  # a tie: equal logits, lower id first
    pos = rng.integers(0, 2**40, rows).astype(np.int64)
    out = la.sample(torch.from_numpy(lg).cuda(), T, k, p, seed,
                    torch.from_numpy(pos).cuda()).cpu().numpy()
    excused = 0
    for r in range(rows):
        t, m = oracle.sample_logits(lg[r], T, k, p, oracle.uniform(seed, int(pos[r])))
        if out[r] != t:
            assert m <= 1e-5, (r, out[r], t, m)
            excused += 1
    log(f"  T={T} k={k} p={p}: {rows} draws, {excused} excused at a boundary")


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.8, 10, 1.0), (1.2, 0, 0.7)])
def test_draw_kernel_distribution(T, k, p):
    rng = np.random.default_rng(21)
    V, n = 40, 30000
    z = rng.normal(0, 1.0, V).astype(np.float32)
    z[7] = z[3]  # equal logits
    lg = torch.from_numpy(np.tile(z, (n, 1))).cuda()
    pos = torch.arange(n, dtype=torch.int64).cuda() + 1000
    out = la.sample(lg, T, k, p, 42, pos).cpu().numpy()
    prob = definition_probs(z, T, k, p)
    counts = np.bincount(out, minlength=V).astype(np.float64)
    keep = prob > 0
    assert counts[~keep].sum() == 0
    e = n * prob[keep]
    chi2 = float(np.sum((counts[keep] - e) ** 2 / e))
    dof = int(keep.sum()) - 1
    crit = dof * (1 - 2 / (9 * dof) + 3.09 * math.sqrt(2 / (9 * dof))) ** 3
    log(f"  T={T} k={k} p={p}: chi2 {chi2:.1f} (dof {dof}, 0.1% critical {crit:.1f})")
    assert chi2 < crit


def test_draw_kernel_rejects_bad_arguments():
    lg = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
    pos = torch.zeros(2, dtype=torch.int64, device="cuda")
    for T, k, p in [(0.0, 0, 1.0), (1.0, -1, 1.0), (1.0, 0, 0.0), (1.0, 0, 1.5)]:
        with pytest.raises(la.LaError):
            la.sample(lg, T, k, p, 0, pos)
    big = torch.zeros((1, 32769), dtype=torch.float32, device="cuda")
    with pytest.raises(la.LaError):
        la.sample(big, 1.0, 0, 1.0, 0, pos[:1])


SAMPLED = [
    (lasynth.get_config("tiny"), (0.9, 0, 1.0, 3), 1e-4),
    (lasynth.get_config("tiny", name="tiny_topk_topp"), (1.2, 20, 0.9, 4), 1e-4),
    (lasynth.get_config("7b", name="bf16_w15", n_layers=3, d_model=512, n_heads=4,
                        n_kv_heads=4, d_ffn=1408, vocab=2048, prompt_len=64,
                        span_len=8, n_spans=2), (0.8, 50, 0.95, 5), 2e-2),
]


@pytest.mark.parametrize("case", SAMPLED, ids=lambda c: c[0].name)
def test_sampled_lockstep(case):
    cfg, sp, tol = case
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p)
    ls = Lockstep(cfg, w, 512, logit_tol=tol, tie_margin=2e-4 if tol < 1e-3 else 0.05,
                  sampling=sp)
    ls.prefill(p, win)
    for _ in range(10):
        ls.step()
    log(f"  {cfg.name} sampled {sp}: max|dlogit|={ls.max_diff:.2e} excused={ls.ties}")


def test_sampled_batch_mixes_greedy_and_sampled():
    cfg = lasynth.get_config("tiny", name="tiny_b3")
    w = lasynth.make_weights(cfg)
    prompts, wins = [], []
    for b, n in enumerate([32, 41, 27]):
        c = cfg.with_(prompt_len=n)
        prompts.append(lasynth.make_prompt(c, seed=b))
        wins.append(lasynth.make_init_window(c, prompts[-1], seed=b))
    ls = BatchLockstep(cfg, w, 1024, 3, logit_tol=1e-4, tie_margin=2e-4,
                       sampling=[None, (0.8, 0, 1.0, 1), (1.1, 15, 0.9, 2)])
    ls.prefill(prompts, wins)
    for _ in range(10):
        ls.step()
    log(f"  mixed batch: max|dlogit|={ls.max_diff:.2e} excused={ls.ties}")


@pytest.mark.parametrize("case", [SAMPLED[0], SAMPLED[2]], ids=lambda c: c[0].name)
def test_sampled_lookahead_equals_plain_sampled(case):
    cfg, sp, tol = case
    T, k, pp, seed = sp
    w = lasynth.make_weights(cfg)
    p = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, p)
    dw = la.upload_weights(w)
    M = 96
    dec = la.LookaheadDecoder(cfg, dw, 1024)
    dec.set_sampling(*sp)
    toks, steps = dec.generate(p, win, M)
    dec.close()
    plain = la.LookaheadDecoder(cfg.with_(W=0, G=0), dw, 1024)
    plain.set_sampling(*sp)
    ref = [plain.prefill(p)]
    margins = [None]
    while len(ref) < M:
        r = plain.step()
        ref += r["tokens"]
        margins.append(oracle.sample_logits(plain.debug_logits()[0], T, k, pp,
                                            oracle.uniform(seed, r["kv_len"]))[1])
    plain.close()
    div = next((i for i in range(M) if toks[i] != ref[i]), None)
    log(f"  {cfg.name}: {len(steps)} steps for {M} tokens, first divergence {div}")
    if div is not None:
        assert div > 0 and margins[div] <= draw_tol(tol, T), (div, margins[div])
