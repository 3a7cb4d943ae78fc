"""Run-to-run determinism of the GPU step (GPU only).

Every sum of the step has a fixed order.
- The reduce kernels add the K-split partials in split order, and the merge
  adds the attention splits in split order.
- Each workgroup walks its K range, or its key chunks, in an order fixed by
  its own index; the rotated starting stages and chunks are included.
- No result goes through an atomic add.

So contexts given the same weights, prompt and window produce bit-identical
logits, tokens, windows, pools and KV caches. This holds on the same GPU,
and for the captured step graph against the same kernels launched directly
(LA_NO_GRAPH=1, read when a context is created). The shape is the full 7B one,
so every kernel instance the step runs at that shape is covered: the K-split
and fused gate/up GEMMs, the per-tile attention, the reduce kernels, and in
plain decode the one-tile GEMMs and the split one-row attention with its merge.
"""
import os

import numpy as np
import pytest
import torch

import lasynth
import lookahead_decoding_la_amd as la
from lockstep import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w7b():
    cfg = lasynth.get_config("7b")
    w = lasynth.make_weights_device(cfg, seed=0)
    torch.cuda.synchronize()
    yield cfg, w
    del w
    torch.cuda.empty_cache()


def _decoder(cfg, w, max_ctx, graph):
    if graph:
        return la.LookaheadDecoder(cfg, w, max_ctx)
    os.environ["LA_NO_GRAPH"] = "1"
    try:
        return la.LookaheadDecoder(cfg, w, max_ctx)
    finally:
        del os.environ["LA_NO_GRAPH"]


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _same_state(ref, other, cfg, label):
    assert np.array_equal(_bits(ref.debug_logits()), _bits(other.debug_logits())), f"{label}: logits"
    assert ref.debug_state() == other.debug_state(), f"{label}: kv length, current token"
    if cfg.W:
        assert np.array_equal(ref.debug_window(), other.debug_window()), f"{label}: window"
        (la_, ta), (lb, tb) = ref.debug_pool(), other.debug_pool()
        assert np.array_equal(la_, lb) and np.array_equal(ta, tb), f"{label}: pool"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("plain", [False, True], ids=["w15n5g15", "plain"])
def test_7b_step_is_bit_reproducible(w7b, plain):
    cfg, w = w7b
    c = cfg.with_(W=0, G=0) if plain else cfg
    prompt = lasynth.make_prompt(c)
    win = lasynth.make_init_window(c, prompt) if c.W else None
    decs = [_decoder(c, w, 1024, graph) for graph in (True, True, False)]
    labels = ["second context", "direct launches"]
    try:
        firsts = [d.prefill(prompt, win) for d in decs]
        assert firsts[1] == firsts[0] and firsts[2] == firsts[0]
        n_steps = 8 if plain else 6
        for i in range(n_steps):
            rs = [d.step() for d in decs]
            for r, lab in zip(rs[1:], labels):
                assert r["tokens"] == rs[0]["tokens"], f"step {i}, {lab}: tokens"
            for d, lab in zip(decs[1:], labels):
                _same_state(decs[0], d, c, f"step {i}, {lab}")
        L = decs[0].debug_state()[0]
        for layer in (0, c.n_layers - 1):
            k0, v0 = decs[0].debug_kv(layer, 0, L)
            for d, lab in zip(decs[1:], labels):
                k1, v1 = d.debug_kv(layer, 0, L)
                assert np.array_equal(_bits(k0), _bits(k1)), f"{lab}: K cache, layer {layer}"
                assert np.array_equal(_bits(v0), _bits(v1)), f"{lab}: V cache, layer {layer}"
        log(f"[determinism] {'plain' if plain else 'W15 N5 G15'}: {n_steps} steps, "
            f"{L} cache positions, three contexts bit-identical")
    finally:
        for d in decs:
            d.close()
