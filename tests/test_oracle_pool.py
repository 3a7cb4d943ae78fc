"""Pin the oracle's n-gram pool: hand-worked insert sequences and a
brute-force list model on random insert streams.

The pages fix no pool policy (parity of the policy itself is unpinned by the
pages); these tests pin the oracle to the policy it states.
"""
import json
import os

import numpy as np
import pytest

import lasynth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ctx(G, N, vocab=16):
    cfg = lasynth.get_config("tiny", n_layers=1, d_model=8, n_heads=1,
                             n_kv_heads=1, head_dim=8, d_ffn=8, vocab=vocab,
                             W=2, N=N, G=G)
    return cfg, oracle.Oracle(cfg, lasynth.make_weights(cfg), 8)


def _lists(cfg, o):
    ln, tl = o.pool()
    return {k: [list(map(int, t)) for t in tl[k][:ln[k]]]
            for k in range(cfg.vocab) if ln[k]}


def test_hand_worked_sequences():
    with open(os.path.join(GOLDEN, "pool_sequences.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        cfg, o = _ctx(c["G"], c["N"])
        for key, tail in c["inserts"]:
            o.pool_insert(key, tail)
        assert _lists(cfg, o) == {int(k): v for k, v in c["expect"].items()}


@pytest.mark.parametrize("G,N", [(1, 2), (2, 3), (3, 2), (5, 5), (4, 4)])
def test_random_streams_match_list_model(G, N):
    cfg, o = _ctx(G, N, vocab=6)
    rng = np.random.default_rng(G * 10 + N)
    model = {}
    for it in range(600):
        key = int(rng.integers(0, 6))
        tail = [int(x) for x in rng.integers(0, 3, size=N - 1)]
        o.pool_insert(key, tail)
        lst = model.setdefault(key, [])
        if tail in lst:
            lst.remove(tail)
        elif len(lst) == G:
            lst.pop(0)
        lst.append(tail)
        if it % 50 == 49:
            assert _lists(cfg, o) == {k: v for k, v in model.items() if v}


def test_seed_pool_hand_worked():
    """Prompt n-gram seeding (Key points, "Ablation"): every N-gram of the
    sequence in position order, with the pool's policy.  Worked by hand for
    N = 3, G = 2 over 5 6 7 5 6 8 5 6 7: the n-grams keyed 5 are (6 7),
    (6 8), (6 7) again, which moves to the newest slot."""
    cfg, o = _ctx(2, 3)
    o.prefill([1, 2], np.zeros((2, 2), np.int32))
    o.seed_pool([5, 6, 7, 5, 6, 8, 5, 6, 7])
    assert _lists(cfg, o) == {5: [[6, 8], [6, 7]], 6: [[7, 5], [8, 5]],
                              7: [[5, 6]], 8: [[5, 6]]}


def test_seed_pool_equals_explicit_inserts():
    cfg, o = _ctx(3, 4, vocab=6)
    cfg2, o2 = _ctx(3, 4, vocab=6)
    seq = [int(x) for x in np.random.default_rng(3).integers(0, 6, size=200)]
    o.seed_pool(seq)
    for p in range(len(seq) - 3):
        o2.pool_insert(seq[p], seq[p + 1:p + 4])
    assert _lists(cfg, o) == _lists(cfg2, o2)
    with pytest.raises(ValueError):
        o.seed_pool([0, 1, 99])
