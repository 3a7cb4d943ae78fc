"""The 13B- and 34B-shaped workloads at full size (GPU only).

LLaMA-2-13B shape (40 layers, d 5120, 40 heads, FFN 13824, W10 N5 G10: 81
rows per step) and the 34B shape with grouped KV heads (48 layers, d 8192,
64 query / 8 KV heads, FFN 22016, W7 N5 G7: 57 rows; about 68 GB of bf16
weights).

- Lockstep with the exact oracle, in the launch shapes bench.py times (its
  default capacity): a 32-token prompt, the pool seeded with the oracle's
  own greedy continuation, two lookahead steps (the first accepts it),
  every valid row's logits and decisions, the result, the window and the
  pool.
- The lookahead output equals plain one-token greedy decoding (both on the
  GPU; 128 generated tokens after a 128-token prompt for 13B, 64 after 64
  for 34B, so that the oracle can check the first divergence): where the
  two runs part, the exact oracle run over the shared history must rank
  both tokens within the decision margin of its best.

Bounds: helpers.full_depth_bounds of the shape (1.5x the rounding-only max
and rms that tests/rounding_bounds.py measures for the bf16 storage on
these weights; decisions excused within 5 sqrt(2) rms of a tie).
"""
import numpy as np
import pytest
import torch

import lasynth
import lookahead_decoding_la_amd as la
import oracle
from helpers import full_depth_bounds
from lockstep import Lockstep, log, margin

pytestmark = pytest.mark.gpu

PLAIN_RUN = {"13b": (128, 128), "34b": (64, 64)}  # prompt tokens, generated tokens

# The capacity bench.py gives these shapes by default (prompt + 105 N + T + 64
# positions): the lockstep runs the launch shapes the benchmark times (at
# 34B, cache rows above 2048 keys, so the split attention kernel).
BENCH_CAPACITY = {"13b": 1024 + 105 * 5 + 81 + 64, "34b": 2048 + 105 * 5 + 57 + 64}


@pytest.fixture(scope="module", params=["13b", "34b"])
def big(request):
    name = request.param
    cfg = lasynth.get_config(name)
    log(f"[{name}] drawing weights on the GPU")
    w = lasynth.make_weights_device(cfg, seed=0)
    torch.cuda.synchronize()
    host = {}
    yield cfg, w, host
    host.clear()
    del w
    torch.cuda.empty_cache()


def _host(big):
    cfg, w, host = big
    if "w" not in host:
        host["w"] = lasynth.host_bits(w)
    return host["w"]


@pytest.mark.timeout(900)
def test_full_size_lockstep_with_oracle(big):
    cfg, dev_w, _ = big
    max_tol, rms_tol, dmargin = full_depth_bounds(cfg.name)
    c32 = cfg.with_(prompt_len=32, n_spans=1, span_len=8, span_repeats=2)
    prompt = [int(x) for x in lasynth.make_prompt(c32)]
    win = lasynth.make_init_window(cfg, np.array(prompt))
    ls = Lockstep(cfg, _host(big), BENCH_CAPACITY[cfg.name], logit_tol=max_tol, tie_margin=dmargin,
                  dev_weights=dev_w)
    first = ls.prefill(prompt, win)
    cont = [ls.orc.greedy_next() for _ in range(cfg.N - 1)]
    ls.orc.rewind(len(prompt), first)
    ls.seed([first] + cont)
    for s in range(2):
        r = ls.step()
        d, rms, ties = ls.step_stats[-1]
        log(f"[{cfg.name}] step {s}: accepted {r['accepted']}, emitted {r['tokens']}, "
            f"max|dlogit| {d:.4f} (bound {max_tol:.3f}), rms {rms:.4f} (bound {rms_tol:.3f}), "
            f"excused decisions {ties}")
    log(f"[{cfg.name}] excused decisions (step, row, oracle margin): {ls.excused}")
    assert ls.rms_diff <= rms_tol
    if not ls.excused:  # the oracle's continuation was the GPU's as well
        assert ls.steps[0]["accepted"] == cfg.N - 1


@pytest.mark.timeout(900)
def test_full_size_lookahead_equals_plain_greedy(big):
    cfg, w, _ = big
    name = cfg.name
    max_tol, _, dmargin = full_depth_bounds(name)
    P, M = PLAIN_RUN[name]
    prompt = lasynth.make_prompt(cfg)[:P]
    win = lasynth.make_init_window(cfg, prompt)
    max_ctx = P + M + cfg.T + 64
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
    plain = la.LookaheadDecoder(cfg.with_(W=0, G=0), w, max_ctx)
    ref = [plain.prefill(prompt)]
    dmax = 0.0
    while len(ref) < M:
        n = len(ref)
        ref += plain.step()["tokens"]
        # same history so far: the two layouts' logits for token n agree
        if n in la_logits and toks[:n] == ref[:n]:
            dmax = max(dmax, float(np.max(np.abs(la_logits[n] - plain.debug_logits()[0]))))
    plain.close()
    div = next((i for i in range(M) if toks[i] != ref[i]), None)
    log(f"[{name}] {len(steps)} lookahead steps; first divergence: {div}; "
        f"max |row-0 logit difference| before it {dmax:.3f}")
    assert dmax <= 2 * max_tol, (dmax, max_tol)
    if div is not None:  # 0: the two contexts' prefills (different launch shapes) part
        orc = oracle.Oracle(cfg, _host(big), P + div + 8)
        _, lo = orc.extend([int(x) for x in prompt] + toks[:div], logits=True)
        z = lo[-1].astype(np.float32)
        gap = [float(z.max() - z[t]) for t in (toks[div], ref[div])]
        log(f"[{name}] at the divergence the oracle ranks the two tokens {gap[0]:.3f} and "
            f"{gap[1]:.3f} below its best (top-2 margin {margin(lo[-1]):.3f})")
        assert max(gap) <= dmargin
