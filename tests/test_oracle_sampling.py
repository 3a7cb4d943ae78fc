"""Pin the oracle's sampled decoding ("Break the Sequential Dependency of LLM
Inference Using Lookahead Decoding", Summary: sampling is supported).

The pages say lookahead decoding supports several sampling schemes but give
no algorithm; the oracle's reading (C source, "sampling"):
  - a draw orders the tokens by logit (descending, lower id first on ties),
    cuts to the top k, weights them by exp((z - z_max) / T), cuts to the
    shortest prefix holding a fraction top_p of the weight, and takes the
    first token whose running weight exceeds u times the total;
  - u for the token at sequence position n comes from Philox4x32-10 keyed
    by the seed with counter n;
  - verification accepts a candidate token exactly when it equals the draw
    at its position.
Pins: the generator's published known-answer vectors; hand-worked draws;
the drawn distribution against the definition's probabilities (quadrature
over u, and a chi-square test on Philox uniforms); sampled lookahead
decoding emitting exactly the tokens of plain sampled decoding (the
property that makes the scheme exact), planted candidates being accepted,
and temperature 0 being greedy.
"""
import json
import math
import os

import numpy as np
import pytest

import lasynth
import oracle
from helpers import definition_probs as _definition_probs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        assert oracle.philox4x32_10(ctr, key) == [int(x, 16) for x in v["out"]]


def test_uniform_is_philox_word0_top_24_bits():
    for seed, pos in [(0, 0), (1, 5), (2**40 + 3, 123456), (7, 2**33 + 1)]:
        w0 = oracle.philox4x32_10([pos & 0xFFFFFFFF, pos >> 32, 0, 0],
                                  [seed & 0xFFFFFFFF, seed >> 32])[0]
        assert oracle.uniform(seed, pos) == (w0 >> 8) / 2.0**24


def test_uniforms_are_uniform():
    u = np.array([oracle.uniform(11, n) for n in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    # Kolmogorov-Smirnov distance, 20000 draws: critical value 1.63/sqrt(n)
    # at the 1% level
    s = np.sort(u)
    d = max(np.max(np.arange(1, s.size + 1) / s.size - s), np.max(s - np.arange(s.size) / s.size))
    assert d < 1.63 / math.sqrt(s.size)


# hand-worked: logits (1, 3, 2, 3): order 1, 3, 2, 0 (ties: lower id
# first); weights at T = 1: 1, 1, e^-1, e^-2, total 2.503214724
LG = [1.0, 3.0, 2.0, 3.0]
TOT = 2.0 + math.exp(-1) + math.exp(-2)


@pytest.mark.parametrize("u,tok", [(0.0, 1), (0.39, 1), (1.0 / TOT - 1e-9, 1),
                                   (1.0 / TOT + 1e-9, 3), (0.79, 3),
                                   (2.0 / TOT + 1e-9, 2), ((2.0 + math.exp(-1)) / TOT + 1e-9, 0),
                                   (0.999, 0)])
def test_draw_hand_worked(u, tok):
    assert oracle.sample_logits(LG, 1.0, u=u)[0] == tok


def test_draw_top_k_and_ties():
    # top 2 = tokens 1 and 3 (equal logits, lower id first), half each
    assert oracle.sample_logits(LG, 1.0, top_k=2, u=0.49)[0] == 1
    assert oracle.sample_logits(LG, 1.0, top_k=2, u=0.51)[0] == 3
    # top 1 of a tie keeps the lower id only
    assert {oracle.sample_logits(LG, 1.0, top_k=1, u=u)[0] for u in (0.0, 0.5, 0.99)} == {1}


def test_draw_top_p():
    # cut 0.3 * TOT < 1: token 1 alone; cut 0.5 * TOT: tokens 1, 3;
    # cut 0.9 * TOT = 2.25 < 2 + e^-1: tokens 1, 3, 2
    assert {oracle.sample_logits(LG, 1.0, top_p=0.3, u=u)[0] for u in (0.0, 0.7, 0.99)} == {1}
    assert oracle.sample_logits(LG, 1.0, top_p=0.5, u=0.99)[0] == 3
    z3 = 2.0 + math.exp(-1)
    assert oracle.sample_logits(LG, 1.0, top_p=0.9, u=(2.0 + 0.5 * math.exp(-1)) / z3)[0] == 2
    assert oracle.sample_logits(LG, 1.0, top_p=0.9, u=0.999)[0] == 2


def test_draw_temperature():
    # T = 0.5: weights e^{2(z - 3)}: 1, 1, e^-2, e^-4 in draw order
    tot = 2.0 + math.exp(-2) + math.exp(-4)
    assert oracle.sample_logits(LG, 0.5, u=(2.0 + 0.5 * math.exp(-2)) / tot)[0] == 2
    assert oracle.sample_logits(LG, 0.5, u=(2.0 + math.exp(-2) + 0.5 * math.exp(-4)) / tot)[0] == 0


SETTINGS = [(1.0, 0, 1.0), (0.7, 0, 1.0), (1.3, 10, 1.0), (1.0, 0, 0.8), (0.9, 25, 0.6)]


@pytest.mark.parametrize("T,k,p", SETTINGS)
def test_draw_distribution_quadrature(T, k, p):
    """u on a grid of midpoints: each token is drawn for a fraction of the
    grid equal to its probability (to the grid spacing)."""
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, 50)
    M = 20000
    counts = np.zeros(50)
    for i in range(M):
        counts[oracle.sample_logits(z, T, k, p, u=(i + 0.5) / M)[0]] += 1
    assert np.max(np.abs(counts / M - _definition_probs(z, T, k, p))) <= 1.0 / M + 1e-12


@pytest.mark.parametrize("T,k,p", SETTINGS[:3])
def test_draw_distribution_philox_chi_square(T, k, p):
    """Draws with the generator's uniforms (one per sequence position)
    against the definition's probabilities: Pearson chi-square below the
    0.1% critical value."""
    rng = np.random.default_rng(5)
    z = rng.normal(0, 1.0, 12)
    prob = _definition_probs(z, T, k, p)
    n = 30000
    counts = np.zeros(12)
    for pos in range(n):
        counts[oracle.sample_logits(z, T, k, p, u=oracle.uniform(99, pos))[0]] += 1
    keep = prob > 0
    assert counts[~keep].sum() == 0
    e = n * prob[keep]
    chi2 = float(np.sum((counts[keep] - e) ** 2 / e))
    dof = int(keep.sum()) - 1
    # Wilson-Hilferty 0.1% critical value
    crit = dof * (1 - 2 / (9 * dof) + 3.09 * math.sqrt(2 / (9 * dof))) ** 3
    assert chi2 < crit, (chi2, crit)


def _sampled(cfg, w, p, win, M, T, k, pp, seed, lookahead=True):
    o = oracle.Oracle(cfg if lookahead else cfg.with_(W=0, G=0), w, 512)
    o.set_sampling(T, k, pp, seed)
    if lookahead:
        return o.generate(p, win, M)
    out = [o.prefill(p)]
    while len(out) < M:
        out.append(o.greedy_next())
    return out, None


@pytest.mark.parametrize("T,k,pp,seed", [(0.8, 0, 1.0, 1), (1.2, 20, 0.9, 2), (0.6, 0, 0.95, 3)])
def test_sampled_lookahead_equals_plain_sampling(tiny, T, k, pp, seed):
    """Every emitted token is the draw at its position from the model's
    distribution given the tokens before it, so lookahead decoding emits
    exactly what plain sampled decoding emits with the same seed."""
    cfg, w, p, win = tiny
    la_out, steps = _sampled(cfg, w, p, win, 64, T, k, pp, seed)
    plain, _ = _sampled(cfg, w, p, win, 64, T, k, pp, seed, lookahead=False)
    assert la_out == plain
    greedy = oracle.Oracle(cfg, w, 512).greedy(p, 64)
    assert la_out != greedy  # the draws are not the argmax


def test_sampled_planted_candidates_are_accepted(tiny):
    """A candidate equal to the continuation the draws produce is accepted
    in full (N - 1 tokens per step)."""
    cfg, w, p, win = tiny
    T, k, pp, seed = 1.0, 0, 1.0, 4
    ref, _ = _sampled(cfg, w, p, win, 40, T, k, pp, seed, lookahead=False)
    o = oracle.Oracle(cfg, w, 512)
    o.set_sampling(T, k, pp, seed)
    out = [o.prefill(p, win)]
    assert out == ref[:1]
    for _ in range(5):
        n = len(out)
        o.pool_insert(out[-1], ref[n:n + cfg.N - 1])
        r = o.step()
        assert r["accepted"] == cfg.N - 1 and r["tokens"] == ref[n:n + cfg.N]
        out += r["tokens"]


def test_temperature_zero_is_greedy(tiny):
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 512)
    o.set_sampling(0.0, 5, 0.5, 9)
    out, _ = o.generate(p, win, 48)
    assert out == oracle.Oracle(cfg, w, 512).greedy(p, 48)


def test_margin_reports_the_boundary_distance():
    # u exactly between the two halves of a 2-token tie: margin 0.5 -> 0
    _, m = oracle.sample_logits([0.0, 0.0], 1.0, u=0.5 - 1e-6)
    assert abs(m - 1e-6) < 1e-9
    _, m = oracle.sample_logits([0.0, 0.0], 1.0, u=0.25)
    assert abs(m - 0.25) < 1e-12
