"""Lockstep comparison of the HIP decoder with the CPU oracle.

Each step the HIP library runs one lookahead step; the oracle forwards the
same block from its own state and takes the same decisions.  Compared:
  - the block tokens (bit-exact);
  - the logits of every valid row (max |diff| <= logit_tol);
  - every row's decision: equal, or else excused: an argmax row whose
    oracle top-2 margin is <= tie_margin, or a drawn row (sampling) whose
    oracle draw margin is <= draw_tol (the draw sat that close to a
    boundary, where logits within logit_tol can move it); the oracle adopts
    the HIP choice and the count is reported;
  - the step result (accepted length, winner, emitted tokens, kv length),
    the window and the n-gram pool (bit-exact).
"""
import sys

import numpy as np

import oracle
import lookahead_decoding_la_amd as la


def margin(row):
    v = np.sort(row.astype(np.float32))
    return float(v[-1]) - float(v[-2])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def draw_tol(logit_tol, temperature):
    """How close to a boundary a draw may sit and still flip when every
    logit may be off by logit_tol: each weight moves by a factor of at most
    exp(logit_tol / T), so a running sum, as a fraction of the total, moves
    by about 2 logit_tol / T; twice that as the excuse."""
    return 4.0 * logit_tol / temperature


class Lockstep:
    def __init__(self, cfg, weights, max_ctx, logit_tol, tie_margin=0.05, sampling=None,
                 storage="exact", dev_weights=None):
        """sampling: (temperature, top_k, top_p, seed) for both sides, or None.
        storage: the oracle's activation storage ("exact" or "bf16").
        dev_weights: device tensors already holding `weights` (else uploaded)."""
        self.cfg = cfg
        self.tol = logit_tol
        self.tie = tie_margin
        if dev_weights is None:
            dev_weights = la.upload_weights(weights)
        self.dev = la.LookaheadDecoder(cfg, dev_weights, max_ctx)
        self.orc = oracle.Oracle(cfg, weights, max_ctx, storage=storage)
        self.sampling = sampling
        if sampling:
            self.dev.set_sampling(*sampling)
            self.orc.set_sampling(*sampling)
        self.ties = 0
        self.max_diff = 0.0
        self.sq_sum, self.n_cmp = 0.0, 0
        self.step_stats = []  # per step: (max |dlogit|, rms |dlogit|, excused ties)
        self.excused = []  # (step, row, oracle margin) of every excused decision
        self.steps = []

    @property
    def rms_diff(self):
        return (self.sq_sum / self.n_cmp) ** 0.5 if self.n_cmp else 0.0

    def _first_token_excused(self, lg, n_prompt, sampling):
        if sampling:
            T, k, p, seed = sampling
            m = oracle.sample_logits(lg[-1], T, k, p, oracle.uniform(seed, n_prompt))[1]
            return m <= draw_tol(self.tol, T), m
        m = margin(lg[-1])
        return m <= self.tie, m

    def prefill(self, prompt, win):
        fg = self.dev.prefill(prompt, win)
        fo, lg = self.orc.prefill(prompt, win, logits=True)
        if fg != fo:
            ok, m = self._first_token_excused(lg, len(prompt), self.sampling)
            assert ok, f"prefill token {fg} vs oracle {fo}, margin {m}"
            self.ties += 1
            self.excused.append((-1, 0, float(m)))
            self.orc.set_current(fg)
        return fg

    def tokens_before_first_excuse(self, out):
        """How many leading tokens of out (the prefill's token, then every
        step's emitted tokens) were decided with no excused decision: all
        of them, or those of the steps before the first that adopted one."""
        if not self.excused:
            return len(out)
        s0 = min(s for s, _, _ in self.excused)
        return 0 if s0 < 0 else 1 + sum(len(r["tokens"]) for r in self.steps[:s0])

    def seed(self, seq):
        """Seed both pools with the n-grams of seq; the pools must agree."""
        self.dev.seed_pool(seq)
        self.orc.seed_pool(seq)
        lg_len, lg_tails = self.dev.debug_pool()
        lo_len, lo_tails = self.orc.pool()
        assert np.array_equal(lg_len, lo_len)
        for key in np.nonzero(lo_len)[0]:
            assert np.array_equal(lg_tails[key][:lo_len[key]], lo_tails[key][:lo_len[key]])

    def step(self):
        rg = self.dev.step()
        lg_g = self.dev.debug_logits()
        tok_g, amax_g = self.dev.debug_block()
        win_g = self.dev.debug_window() if self.cfg.W else None
        pool_g = self.dev.debug_pool() if self.cfg.G else None
        self._compare(self.orc, rg, lg_g, tok_g, amax_g, win_g, pool_g,
                      self.dev.debug_state(), self.sampling)
        self.steps.append(rg)
        return rg

    def _compare(self, orc, rg, lg_g, tok_g, amax_g, win_g, pool_g, state_g, sampling=None):
        """One sequence's step on the device (its rows' logits, tokens and
        argmax, result, window, pool, state) against the oracle stepping the
        same block from its own state."""
        cfg = self.cfg
        tok_o, valid, nc = orc.block_tokens()
        v = valid.astype(bool)
        assert nc == rg["n_candidates"], (nc, rg)
        assert np.array_equal(tok_g[v], tok_o[v])
        lg_o = orc.forward_block(tok_o, valid, keep=True)
        diff = lg_g[v].astype(np.float64) - lg_o[v]
        d = float(np.max(np.abs(diff)))
        sq = float(np.sum(diff * diff))
        self.max_diff = max(self.max_diff, d)
        self.sq_sum += sq
        self.n_cmp += diff.size
        ties0 = self.ties
        assert d <= self.tol, f"logit diff {d} > {self.tol} at step {len(self.steps)}"
        amax_o, dmarg = orc.block_select()
        for r in np.nonzero(v)[0]:
            if amax_g[r] != amax_o[r]:
                if np.isnan(dmarg[r]):
                    m, lim = margin(lg_o[r]), self.tie
                else:
                    m, lim = dmarg[r], draw_tol(self.tol, sampling[0])
                assert m <= lim, (
                    f"step {len(self.steps)} row {r}: token {amax_g[r]} vs oracle "
                    f"{amax_o[r]}, oracle margin {m}")
                self.ties += 1
                self.excused.append((len(self.steps), int(r), float(m)))
                amax_o[r] = amax_g[r]
        self.step_stats.append((d, (sq / diff.size) ** 0.5, self.ties - ties0))
        ro = orc.commit(amax_o)
        assert ro == rg, (ro, rg)
        if cfg.W:
            assert np.array_equal(win_g, orc.window())
        if cfg.G:
            lg_len, lg_tails = pool_g
            lo_len, lo_tails = orc.pool()
            assert np.array_equal(lg_len, lo_len)
            mask = np.arange(cfg.G)[None, :] < lo_len[:, None]
            assert np.array_equal(lg_tails[mask], lo_tails[mask])
        assert state_g == (orc.kv_len, orc.current)

    def run(self, prompt, win, n_steps=None, M=None):
        out = [self.prefill(prompt, win)]
        while (n_steps is None or len(self.steps) < n_steps) and (M is None or len(out) < M):
            out += self.step()["tokens"]
        return out

    def compare_kv(self, tol):
        L = self.orc.kv_len
        for layer in range(self.cfg.n_layers):
            kg, vg = self.dev.debug_kv(layer, 0, L)
            ko, vo = self.orc.kv(layer, 0, L)
            assert np.max(np.abs(kg - ko)) <= tol
            assert np.max(np.abs(vg - vo)) <= tol


class BatchLockstep(Lockstep):
    """B sequences stepped together by one HIP context (one forward pass of
    B blocks), each compared with an oracle of its own: a batched step is B
    independent single-sequence steps."""

    def __init__(self, cfg, weights, max_ctx, B, logit_tol, tie_margin=0.05, sampling=None):
        """sampling: per-sequence list of (temperature, top_k, top_p, seed)
        or None entries (greedy), or None for an all-greedy batch."""
        self.cfg = cfg
        self.B = B
        self.tol = logit_tol
        self.tie = tie_margin
        self.dev = la.LookaheadDecoder(cfg, la.upload_weights(weights), max_ctx, batch=B)
        self.orcs = [oracle.Oracle(cfg, weights, max_ctx) for _ in range(B)]
        self.seq_sampling = list(sampling) if sampling else [None] * B
        for b, sp in enumerate(self.seq_sampling):
            if sp:
                self.dev.set_sampling(*sp, seq=b)
                self.orcs[b].set_sampling(*sp)
        self.ties = 0
        self.max_diff = 0.0
        self.sq_sum, self.n_cmp = 0.0, 0
        self.step_stats = []
        self.excused = []
        self.steps = []

    def prefill(self, prompts, wins):
        return [self.prefill_one(b, prompts[b], wins[b]) for b in range(self.B)]

    def prefill_one(self, b, prompt, win):
        """(Re)start sequence b alone, on the device and in its oracle."""
        fg = self.dev.prefill(prompt, win, seq=b)
        fo, lg = self.orcs[b].prefill(prompt, win, logits=True)
        if fg != fo:
            ok, m = self._first_token_excused(lg, len(prompt), self.seq_sampling[b])
            assert ok, f"seq {b} prefill token {fg} vs oracle {fo}, margin {m}"
            self.ties += 1
            self.orcs[b].set_current(fg)
        return fg

    def step(self):
        cfg, T = self.cfg, self.dev.T
        rgs = self.dev.step()
        lg_g = self.dev.debug_logits()
        tok_g, amax_g = self.dev.debug_block()
        win_g = self.dev.debug_window() if cfg.W else None
        pool_g = self.dev.debug_pool() if cfg.G else None
        states = self.dev.debug_state()
        for b in range(self.B):
            rows = slice(b * T, (b + 1) * T)
            self._compare(self.orcs[b], rgs[b], lg_g[rows], tok_g[rows], amax_g[rows],
                          win_g[b] if cfg.W else None,
                          (pool_g[0][b], pool_g[1][b]) if cfg.G else None, states[b],
                          self.seq_sampling[b])
        self.steps.append(rgs)
        return rgs

    def compare_kv(self, tol):
        # one copy of every sequence's cache rows per layer (la_debug_kv
        # returns the whole batch), up to the longest committed length
        Lmax = max(orc.kv_len for orc in self.orcs)
        for layer in range(self.cfg.n_layers):
            kg, vg = self.dev.debug_kv(layer, 0, Lmax)
            if self.B == 1:  # the binding drops the batch axis of one sequence
                kg, vg = kg[None], vg[None]
            for b, orc in enumerate(self.orcs):
                L = orc.kv_len
                ko, vo = orc.kv(layer, 0, L)
                assert np.max(np.abs(kg[b][:, :L] - ko)) <= tol
                assert np.max(np.abs(vg[b][:, :L] - vo)) <= tol
