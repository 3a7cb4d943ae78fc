"""Pin the oracle's lookahead step to what the paper and arithmetic fix.

- Output invariance (Summary: the verification branch keeps the output
  distribution unchanged): under greedy decoding, lookahead decoding must emit
  exactly the plain one-token-at-a-time greedy tokens.
- Every block row's logits must equal a from-scratch causal run over the
  token sequence that row can see (the mask's implied sequence).
- Rows per step 1 + (W+G)(N-1) against the paper's extra-work multiples.
- Planted candidates, empty pool, W = G = 0 and mask-isolation special cases.
"""
import json
import os

import numpy as np
import pytest

import lasynth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _setup(cfg, seed=0, ctx=256):
    w = lasynth.make_weights(cfg, seed=seed)
    p = lasynth.make_prompt(cfg, seed=seed)
    win = lasynth.make_init_window(cfg, p, seed=seed) if cfg.W else None
    return w, p, win


VARIANTS = [
    lasynth.get_config("tiny"),
    lasynth.get_config("tiny", name="n2", N=2),
    lasynth.get_config("tiny", name="n5", N=5, W=3, G=4),
    lasynth.get_config("tiny", name="verify_only", W=0, G=3),
    lasynth.get_config("tiny", name="lookahead_only", W=4, G=0),
    lasynth.get_config("tiny", name="bf16_gqa", dtype="bf16", d_model=64,
                       n_heads=4, n_kv_heads=2, head_dim=16, d_ffn=96,
                       vocab=300, W=4, N=4, G=3),
]


@pytest.mark.parametrize("cfg", VARIANTS, ids=lambda c: c.name)
def test_lookahead_tokens_equal_greedy(cfg):
    w, p, win = _setup(cfg)
    M = 64
    a = oracle.Oracle(cfg, w, 256)
    toks, steps = a.generate(p, win, M)
    b = oracle.Oracle(cfg, w, 256)
    assert toks == b.greedy(p, M)
    assert all(1 <= s["n_emitted"] <= cfg.N for s in steps)


def test_tiny_lookahead_accepts_multiple_tokens(tiny):
    # The motif-repeating prompt lets the pool find the greedy continuation.
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 256)
    _, steps = o.generate(p, win, 64)
    assert sum(s["n_emitted"] for s in steps) / len(steps) > 1.2


def _implied(cfg, r, tok):
    """Tokens of the block rows row r sees, in position order (via the mask)."""
    vis = [s for s in range(cfg.T) if oracle.visible(cfg, r, s)]
    vis.sort(key=lambda s: oracle.row_pos(cfg, s))
    return vis, [int(tok[s]) for s in vis]


@pytest.mark.parametrize("cfg", VARIANTS[:3], ids=lambda c: c.name)
def test_block_rows_equal_causal_rerun(cfg):
    w, p, win = _setup(cfg)
    o = oracle.Oracle(cfg, w, 256)
    gen = [o.prefill(p, win)]
    for step in range(8):
        tok, valid, nc = o.block_tokens()
        L = o.kv_len
        committed = (list(p) + gen)[:L]
        lg = o.forward_block(tok, valid, keep=True)
        for r in range(cfg.T):
            if not valid[r]:
                assert np.all(np.isnan(lg[r]))
                continue
            rows, seq = _implied(cfg, r, tok)
            # every visible row is valid, positions are exactly 0..p_r
            assert all(valid[s] for s in rows)
            assert [oracle.row_pos(cfg, s) for s in rows] == list(
                range(oracle.row_pos(cfg, r) + 1))
            ref = oracle.Oracle(cfg, w, 256)
            _, rl = ref.extend(committed + seq, logits=True)
            assert np.array_equal(rl[-1], lg[r]), (step, r)
        res = o.commit()
        gen += res["tokens"]
        # committed KV equals a causal run over the committed tokens
        ref = oracle.Oracle(cfg, w, 256)
        ref.extend((list(p) + gen)[:o.kv_len])
        for layer in range(cfg.n_layers):
            ka, va = o.kv(layer, 0, o.kv_len)
            kb, vb = ref.kv(layer, 0, o.kv_len)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_mask_matches_window_trajectories(tiny):
    """Row (l, j) sees cur, win[1][0..j], win[2][j], ..., win[l][j]; row
    (g, i) sees cur, cand[g][0..i-1]: the 2D window's diagonals."""
    cfg = tiny[0]
    for cfg in (cfg, VARIANTS[2], VARIANTS[1]):
        W, n1 = cfg.W, cfg.N - 1
        tok = np.arange(cfg.T, dtype=np.int32) + 1000  # row r holds token 1000+r
        def la(l, j):
            return 1 + (l - 1) * W + j
        def cd(g, i):
            return 1 + n1 * W + g * n1 + (i - 1)
        for l in range(1, n1 + 1):
            for j in range(W):
                want = [0] + [la(1, jj) for jj in range(j + 1)] + [la(ll, j) for ll in range(2, l + 1)]
                assert _implied(cfg, la(l, j), tok)[0] == want
        for g in range(cfg.G):
            for i in range(1, n1 + 1):
                want = [0] + [cd(g, ii) for ii in range(1, i + 1)]
                assert _implied(cfg, cd(g, i), tok)[0] == want
        assert _implied(cfg, 0, tok)[0] == [0]


def test_mask_isolation(tiny):
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 256)
    o.prefill(p, win)
    for _ in range(3):
        o.step()
    rng = np.random.default_rng(1)
    for _ in range(3):  # plant candidates under the current token
        o.pool_insert(o.current, rng.integers(0, cfg.vocab, size=cfg.N - 1))
    tok, valid, nc = o.block_tokens()
    assert nc >= 3
    base = o.forward_block(tok, valid, keep=False)
    W, n1 = cfg.W, cfg.N - 1
    la_rows = list(range(0, 1 + W * n1))
    cand = lambda g: [1 + n1 * W + g * n1 + i for i in range(n1)]
    # perturb every candidate: row 0 and lookahead rows unchanged
    t2 = tok.copy()
    for g in range(nc):
        for r in cand(g):
            t2[r] = (t2[r] + 7) % cfg.vocab
    lg = o.forward_block(t2, valid, keep=False)
    assert np.array_equal(lg[la_rows], base[la_rows])
    assert not np.array_equal(lg[cand(0)], base[cand(0)])
    # perturb candidate 0: the other candidates unchanged
    t3 = tok.copy()
    t3[cand(0)[0]] = (t3[cand(0)[0]] + 1) % cfg.vocab
    lg = o.forward_block(t3, valid, keep=False)
    for g in range(1, nc):
        assert np.array_equal(lg[cand(g)], base[cand(g)])
    assert np.array_equal(lg[la_rows], base[la_rows])
    # perturb window entry (l, j): only (l' >= l, j) change, and for l = 1
    # also every (l', j' >= j)
    for (l, j) in [(1, 2), (2, 1), (2, 4), (1, 0)]:
        r0 = 1 + (l - 1) * W + j
        t4 = tok.copy()
        t4[r0] = (t4[r0] + 3) % cfg.vocab
        lg = o.forward_block(t4, valid, keep=False)
        for ll in range(1, n1 + 1):
            for jj in range(W):
                r = 1 + (ll - 1) * W + jj
                hit = (jj == j and ll >= l) or (l == 1 and jj >= j)
                assert np.array_equal(lg[r], base[r]) != hit, (l, j, ll, jj)
        assert np.array_equal(lg[0], base[0])


def test_rows_per_step_match_paper_extra_work():
    with open(os.path.join(GOLDEN, "step_rows.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        W, N, G = case["W"], case["N"], case["G"]
        assert (W + G) * (N - 1) == case["extra_rows"]
        cfg = lasynth.get_config(case["config"])
        assert (cfg.W, cfg.N, cfg.G) == (W, N, G)
        assert cfg.T == 1 + case["extra_rows"]
        o_cfg = cfg.with_(n_layers=1, d_model=8, n_heads=1, n_kv_heads=1,
                          head_dim=8, d_ffn=8, vocab=16, dtype="f32")
        w = lasynth.make_weights(o_cfg)
        assert oracle.Oracle(o_cfg, w, 4 * cfg.T).T == cfg.T


def test_planted_candidate_is_accepted(tiny):
    cfg, w, p, win = tiny
    M = 40
    greedy = oracle.Oracle(cfg, w, 256).greedy(p, M)
    o = oracle.Oracle(cfg, w, 256)
    out = [o.prefill(p, win)]
    for step in range(6):
        cur = o.current
        assert out[-1] == cur
        n = len(out)
        # true continuation of the current token
        o.pool_insert(cur, greedy[n:n + cfg.N - 1])
        r = o.step()
        assert r["accepted"] == cfg.N - 1
        assert r["n_emitted"] == cfg.N
        assert r["tokens"] == greedy[n:n + cfg.N]
        out += r["tokens"]


def test_empty_pool_emits_one_token(tiny):
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 256)
    first = o.prefill(p, win)
    r = o.step()
    assert r["n_candidates"] == 0 and r["winner"] == -1
    assert r["n_emitted"] == 1 and r["accepted"] == 0
    g = oracle.Oracle(cfg, w, 256)
    g.prefill(p, win)
    assert r["tokens"] == [g.greedy_next()]
    assert r["kv_len"] == len(p) + 1


def test_plain_step_equals_greedy_step(tiny):
    cfg, w, p, _ = tiny
    c0 = cfg.with_(W=0, G=0)
    a = oracle.Oracle(c0, w, 256)
    b = oracle.Oracle(c0, w, 256)
    a.prefill(p)
    b.prefill(p)
    assert a.T == 1
    for _ in range(20):
        r, la = a.step(logits=True)
        t, lb = b.greedy_next(logits=True)
        assert np.array_equal(la[0], lb)
        assert r["tokens"] == [t] and r["winner"] == -1


def test_window_shift_and_pool_update(tiny):
    """After a step: level l becomes the old level l+1, the new last level is
    the last level's argmax, and the pool holds the column n-grams."""
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 256)
    o.prefill(p, win)
    model = {}
    for _ in range(10):
        w0 = o.window()
        tok, valid, nc = o.block_tokens()
        o.forward_block(tok, valid, keep=True)
        amax = o.block_argmax()
        o.commit()
        n1, W = cfg.N - 1, cfg.W
        ynew = [int(amax[1 + (n1 - 1) * W + j]) for j in range(W)]
        w1 = o.window()
        assert np.array_equal(w1[:-1], w0[1:])
        assert list(w1[-1]) == ynew
        for j in range(W):
            tail = [int(w0[l][j]) for l in range(1, n1)] + [ynew[j]]
            lst = model.setdefault(int(w0[0][j]), [])
            if tail in lst:
                lst.remove(tail)
            elif len(lst) == cfg.G:
                lst.pop(0)
            lst.append(tail)
        ln, tl = o.pool()
        for key in range(cfg.vocab):
            assert ln[key] == len(model.get(key, []))
            assert [list(map(int, t)) for t in tl[key][:ln[key]]] == model.get(key, [])


def test_prompt_seeded_pool_keeps_greedy_output(tiny):
    """With the pool seeded from the prompt (Key points, "Ablation") the
    output is still plain greedy decoding: seeding changes which candidates
    are verified, never what is emitted."""
    cfg, w, p, win = tiny
    M = 48
    ref = oracle.Oracle(cfg, w, 256).greedy(p, M)
    toks, steps = oracle.Oracle(cfg, w, 256).generate(p, win, M, seed_prompt=True)
    assert toks == ref
    assert all(1 <= s["n_emitted"] <= cfg.N for s in steps)


def _plant(o, cfg, tails):
    for t in tails:
        o.pool_insert(o.current, np.asarray(t, np.int32))


def test_argmax_equals_numpy_argmax_of_fp32_logits(tiny):
    """Every valid row's decision in a greedy step is numpy.argmax of that
    row's logits rounded to fp32 (numpy returns the first, i.e. lowest-id,
    maximum); invalid candidate slots carry -1."""
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 256)
    o.prefill(p, win)
    rng = np.random.default_rng(3)
    seen_invalid = False
    for step in range(4):
        _plant(o, cfg, [rng.integers(0, cfg.vocab, cfg.N - 1) for _ in range(step % 3)])
        tok, valid, nc = o.block_tokens()
        lg = o.forward_block(tok, valid, keep=True)
        amax = o.block_argmax()
        for r in range(cfg.T):
            if valid[r]:
                assert amax[r] == int(np.argmax(lg[r].astype(np.float32))), (step, r)
            else:
                seen_invalid = True
                assert amax[r] == -1
        o.commit()
    assert seen_invalid


def test_argmax_ties_take_the_lowest_token_id(tiny):
    """Exact ties built into the weights: an LM head whose rows are all zero
    except three identical rows (ids 5, 17, 300).  Every row's logits are
    then exactly 0 except three bit-identical values z; the decision must be
    5 where z > 0 and 0 (the lowest id among the zeros) where z <= 0.  A
    highest-id rule, or a reversed comparison, fails here."""
    cfg, w, p, win = tiny
    w2 = [x.copy() for x in w]
    lm = w2[2]
    assert lm.shape == (cfg.vocab, cfg.d_model)
    lm[:] = 0
    row = np.random.default_rng(11).normal(0.0, 0.5, cfg.d_model).astype(lm.dtype)
    for t in (5, 17, 300):
        lm[t] = row
    o = oracle.Oracle(cfg, w2, 256)
    first, lgp = o.prefill(p, win, logits=True)
    z = lgp[-1][5]
    assert lgp[-1][17] == z and lgp[-1][300] == z
    assert first == (5 if np.float32(z) > 0 else 0)
    signs = set()
    for _ in range(3):
        _plant(o, cfg, [[5] * (cfg.N - 1), [0] * (cfg.N - 1)])
        tok, valid, nc = o.block_tokens()
        lg = o.forward_block(tok, valid, keep=True)
        amax = o.block_argmax()
        for r in np.nonzero(valid)[0]:
            zr = lg[r][5]
            others = np.delete(lg[r], [5, 17, 300])
            assert np.all(others == 0.0) and lg[r][17] == zr and lg[r][300] == zr
            want = 5 if np.float32(zr) > 0 else 0
            signs.add(want)
            assert amax[r] == want, (r, zr)
        o.commit()
    assert signs, "no valid rows"


def _verify_case(tiny, tails, decide):
    """Plant `tails` under the current token, forward the block, then commit
    with the decisions `decide(row_of_candidate, amax)` fixes on top of the
    oracle's own argmax; returns (result, block tokens)."""
    cfg, w, p, win = tiny
    o = oracle.Oracle(cfg, w, 256)
    o.prefill(p, win)
    _plant(o, cfg, tails)
    tok, valid, nc = o.block_tokens()
    assert nc == len(tails)
    o.forward_block(tok, valid, keep=True)
    amax = o.block_argmax()
    n1, W = cfg.N - 1, cfg.W

    def cand_row(g, i):  # row of candidate g's token i (1-based)
        return 1 + n1 * W + g * n1 + (i - 1)

    decide(cand_row, amax)
    return o.commit(amax), tok


def test_winner_is_lowest_index_among_equal_accepted_lengths(tiny):
    """Hand-worked verification (N = 3, two candidate tokens each):
    candidates (a, b) and (a, c) both accept k = 2 when row 0 decides a and
    both candidates' first rows decide their second tokens; the winner is
    candidate 0, and the bonus token is the decision of candidate 0's last
    row."""
    cfg = tiny[0]
    assert cfg.N == 3 and cfg.G >= 3
    a, b, c = 7, 8, 9

    def decide(row, amax):
        amax[0] = a
        amax[row(0, 1)] = b   # cand 0: a, b -> k = 2
        amax[row(1, 1)] = c   # cand 1: a, c -> k = 2
        amax[row(0, 2)] = 41  # bonus of cand 0
        amax[row(1, 2)] = 42  # bonus of cand 1
    res, _ = _verify_case(tiny, [[a, b], [a, c]], decide)
    assert res["accepted"] == 2 and res["winner"] == 0
    assert res["tokens"] == [a, b, 41] and res["n_emitted"] == 3


def test_winner_is_the_longest_accepted_prefix(tiny):
    """A later candidate with a longer accepted prefix wins: (a, x) accepts
    1, (a, b) accepts 2 -> winner 1, emits a, b and candidate 1's bonus."""
    a, b, x = 7, 8, 9

    def decide(row, amax):
        amax[0] = a
        amax[row(0, 1)] = b   # cand 0 is (a, x): stops after a
        amax[row(1, 1)] = b   # cand 1 is (a, b): accepts both
        amax[row(0, 2)] = 50
        amax[row(1, 2)] = 51
    res, _ = _verify_case(tiny, [[a, x], [a, b]], decide)
    assert res["accepted"] == 2 and res["winner"] == 1
    assert res["tokens"] == [a, b, 51]


def test_winner_with_nothing_accepted_is_candidate_zero(tiny):
    """No candidate's first token equals row 0's decision: k = 0, the winner
    is candidate 0 (candidates were present), one token is emitted (row 0's
    decision); with three candidates of k = 1, 1, 0 the winner is 0."""
    a = 7

    def none(row, amax):
        amax[0] = a
    res, _ = _verify_case(tiny, [[1, 2], [3, 4], [5, 6]], none)
    assert res["accepted"] == 0 and res["winner"] == 0
    assert res["tokens"] == [a] and res["n_candidates"] == 3

    def ones(row, amax):
        amax[0] = a
        amax[row(0, 1)] = 99  # cand 0 (a, 2): k = 1
        amax[row(1, 1)] = 98  # cand 1 (a, 4): k = 1
    res, _ = _verify_case(tiny, [[a, 2], [a, 4], [5, 6]], ones)
    assert res["accepted"] == 1 and res["winner"] == 0
    assert res["tokens"] == [a, 99]


def test_rewind_then_decode_again_is_identical(tiny):
    """Decoding ahead with plain greedy steps and rewinding to the prefill
    state leaves the context as a fresh prefill would: the next lookahead
    step's result and logits are unchanged."""
    cfg, w, p, win = tiny
    a = oracle.Oracle(cfg, w, 256)
    first = a.prefill(p, win)
    ahead = [a.greedy_next() for _ in range(6)]
    assert ahead == oracle.Oracle(cfg, w, 256).greedy(p, 7)[1:]
    a.rewind(len(p), first)
    ra, la_ = a.step(logits=True)
    b = oracle.Oracle(cfg, w, 256)
    b.prefill(p, win)
    rb, lb = b.step(logits=True)
    assert ra == rb and np.array_equal(la_, lb, equal_nan=True)
    with pytest.raises(ValueError):
        a.rewind(a.kv_len + 1, 0)


def test_prefill_in_chunks_equals_one_prefill(tiny):
    """A prompt prefilled as a first chunk (with the window), the rest appended
    causally with extend, and the current token set to the decision after the
    last prompt token, leaves the same state as one prefill: the same current
    token and KV cache, and the next lookahead step's block and logits are
    identical (bench.py's CPU baseline prefills long prompts this way)."""
    cfg, w, p, win = tiny
    p = [int(x) for x in p]
    a = oracle.Oracle(cfg, w, 256)
    b = oracle.Oracle(cfg, w, 256)
    ta = a.prefill(p, win)
    tb = b.prefill(p[:5], win)
    for s in range(5, len(p), 7):
        tb = b.extend(p[s:s + 7])
    b.set_current(tb)
    assert ta == tb
    for layer in range(cfg.n_layers):
        for kh in range(cfg.n_kv_heads):
            ka, va = a.kv(layer, kh, len(p))
            kb, vb = b.kv(layer, kh, len(p))
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    tok_a, val_a, nc_a = a.block_tokens()
    tok_b, val_b, nc_b = b.block_tokens()
    assert nc_a == nc_b and np.array_equal(tok_a, tok_b) and np.array_equal(val_a, val_b)
    v = val_a.astype(bool)
    la_ = a.forward_block(tok_a, val_a, keep=False)
    lb_ = b.forward_block(tok_b, val_b, keep=False)
    assert np.array_equal(la_[v], lb_[v])
