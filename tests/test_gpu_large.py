"""The 13B- and 34B-shaped workloads at full size (GPU only).

LLaMA-2-13B shape (40 layers, d 5120, 40 heads, FFN 13824, W10 N5 G10: 81
rows per step) and the 34B shape with grouped KV heads (48 layers, d 8192,
64 query / 8 KV heads, FFN 22016, W7 N5 G7: 57 rows; about 68 GB of bf16
weights).  The narrow versions of these step shapes run in lockstep with the
oracle in tests/test_gpu_parity.py; here the full models are checked
through a property that holds at any size: lookahead decoding emits the
tokens of plain one-token greedy decoding on the same weights (both on the
GPU).  Up to the first divergence the two runs share the history, so a
lookahead step's current-token row and the plain step at the same position
compute the same logits through different row layouts; each is within the
shape's full-depth bound of the exact logits (1.5x the rounding-only error
that tests/rounding_bounds.py measures on these weights: 0.293 for 13B,
0.679 for 34B), so they must agree within twice it, and the divergence
must sit where the plain run's top-2 margin is within twice that.
"""
import numpy as np
import pytest
import torch

import lasynth
import lookahead_decoding_la_amd as la
from helpers import full_depth_logit_tol
from lockstep import log, margin

pytestmark = pytest.mark.gpu

M = 128  # generated tokens (the prefill's included)


@pytest.mark.parametrize("name", ["13b", "34b"])
def test_full_size_lookahead_equals_plain_greedy(name):
    cfg = lasynth.get_config(name)
    log(f"[{name}] drawing weights on the GPU")
    w = lasynth.make_weights_device(cfg, seed=0)
    torch.cuda.synchronize()
    prompt = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, prompt)
    max_ctx = cfg.prompt_len + M + cfg.T + 64
    dec = la.LookaheadDecoder(cfg, w, max_ctx)
    toks = [dec.prefill(prompt, win)]
    steps, la_logits = [], {}  # position of the token a step's row 0 predicts -> logits
    while len(toks) < M:
        r = dec.step()
        la_logits[len(toks)] = dec.debug_logits()[0].copy()
        steps.append(r)
        toks += r["tokens"]
    toks = toks[:M]
    dec.close()
    acc = sum(s["n_emitted"] for s in steps) / len(steps)
    log(f"[{name}] lookahead: {len(steps)} steps for {M} tokens ({acc:.2f} tokens/step)")
    plain = la.LookaheadDecoder(cfg.with_(W=0, G=0), w, max_ctx)
    ref = [plain.prefill(prompt)]
    margins, dmax = [None], 0.0
    while len(ref) < M:
        n = len(ref)
        ref += plain.step()["tokens"]
        lg = plain.debug_logits()[0]
        margins.append(margin(lg))
        # same history so far: the two layouts' logits for token n agree
        if n in la_logits and toks[:n] == ref[:n]:
            dmax = max(dmax, float(np.max(np.abs(la_logits[n] - lg))))
    plain.close()
    del w
    torch.cuda.empty_cache()
    div = next((i for i in range(M) if toks[i] != ref[i]), None)
    log(f"[{name}] first divergence: {div}" +
        (f" (plain margin {margins[div]:.3f})" if div else "") +
        f"; max |logit difference| before it {dmax:.3f}")
    tol = full_depth_logit_tol(name)
    assert dmax <= 2 * tol, (dmax, tol)
    if div is not None:
        assert div > 0 and margins[div] <= 4 * tol, (div, margins[div])
