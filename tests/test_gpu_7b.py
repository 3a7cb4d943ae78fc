"""The LLaMA-2-7B-shaped workload at full size (GPU only), in the launch
configuration bench.py times (121 rows per step, W15 N5 G15).

- Headline lockstep: from the workload's 512-token prompt, six lookahead
  steps in lockstep with the exact oracle, the pool seeded with the prompt's
  n-grams and with the oracle's own greedy continuation, so that steps
  accept candidates (KV compaction, multi-token emits).  Every step: all
  valid rows' logits, every decision, the block tokens, the step result,
  the window and the whole pool.
- A property that holds at any size: the lookahead output equals plain
  one-token greedy decoding (both on the GPU, 512-token prompt, 256
  tokens); where the two runs part, the exact oracle (run over the shared
  history) must rank both tokens within the decision margin of its best.

Bounds at full depth (bf16 datapath against exact arithmetic; see
helpers.full_depth_bounds).  The datapath stores seven activations per layer
in bf16; that storage alone moves this model's logits by up to 0.185 (rms
0.034) on its own weights (tests/rounding_bounds.py, all seven points; by
point alone the KV cache and q/k/v move them most, 0.124).  No bf16
reference helps here: a bf16-storage oracle rounding at the very same
points differs from this datapath by as much as the exact oracle does, since
two bf16 pipelines' rounding errors decorrelate within a few layers once
their inputs differ by a fraction of a bf16 step.  The tests therefore hold
every logit to 1.5x the rounding-only max (0.278), the rms difference to
1.5x the rounding-only rms (0.051), and excuse a differing decision only
where the oracle's top-2 margin is within 5 sqrt(2) times that rms (0.24).
The 2e-2 logit bound and 0.05 decision margin hold on the shallow bf16
configurations (tests/test_gpu_parity.py), not at 32 layers.
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

MAX_TOL, RMS_TOL, DECISION_MARGIN = full_depth_bounds("7b")


@pytest.fixture(scope="module")
def w7b():
    cfg = lasynth.get_config("7b")
    log("[7b] drawing weights on the GPU")
    w = lasynth.make_weights_device(cfg, seed=0)
    torch.cuda.synchronize()
    yield cfg, w
    del w
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_7b_headline_lockstep(w7b):
    cfg, dev_w = w7b
    prompt = [int(x) for x in lasynth.make_prompt(cfg)]
    win = lasynth.make_init_window(cfg, np.array(prompt))
    assert len(prompt) == 512 and cfg.T == 121
    ls = Lockstep(cfg, lasynth.host_bits(dev_w), 1024, logit_tol=MAX_TOL,
                  tie_margin=DECISION_MARGIN, dev_weights=dev_w)
    log("[7b] prefill of 512 tokens, GPU and oracle")
    first = ls.prefill(prompt, win)
    # the oracle's own greedy continuation (14 tokens: three accepting
    # steps of N - 1 = 4 candidates plus a bonus each), then back
    cont = [ls.orc.greedy_next() for _ in range(14)]
    ls.orc.rewind(len(prompt), first)
    ls.seed(prompt)
    ls.seed([first] + cont)
    for s in range(6):
        r = ls.step()
        d, rms, ties = ls.step_stats[-1]
        log(f"[7b] step {s}: accepted {r['accepted']}, emitted {r['tokens']}, "
            f"max|dlogit| {d:.4f}, rms {rms:.4f}, excused decisions {ties}")
    far = [m for _, _, m in ls.excused if m > 0.05]
    log(f"[7b] lockstep: max|dlogit| {ls.max_diff:.4f} (bound {MAX_TOL:.3f}), "
        f"rms {ls.rms_diff:.4f} (bound {RMS_TOL:.3f}), {ls.ties} excused decisions of "
        f"1 + 6 x {cfg.T} decisions; "
        f"{len(far)} of them at oracle margins above 0.05 {sorted(far)}")
    assert ls.rms_diff <= RMS_TOL
    assert sum(st["accepted"] for st in ls.steps) >= cfg.N - 1
    # KV compaction: layer 0's cache (whose rows depend on nothing but the
    # token, its position and layer-0 weights) holds the right rows
    kg, vg = ls.dev.debug_kv(0, 0, ls.orc.kv_len)
    ko, vo = ls.orc.kv(0, 0, ls.orc.kv_len)
    for g, o in ((kg, ko), (vg, vo)):
        assert np.all(np.abs(g - o) <= 2.0 ** -7 * np.abs(o) + 2e-3)


@pytest.mark.timeout(900)
def test_7b_lookahead_output_equals_plain_greedy(w7b):
    cfg, dev_w = w7b
    prompt = lasynth.make_prompt(cfg)
    win = lasynth.make_init_window(cfg, prompt)
    M = cfg.gen_tokens
    dec = la.LookaheadDecoder(cfg, dev_w, 1024)
    toks = [dec.prefill(prompt, win)]
    steps, la_logits = [], {}  # position of the token a step's row 0 predicts -> logits
    while len(toks) < M:
        r = dec.step()
        la_logits[len(toks)] = dec.debug_logits()[0].copy()
        steps.append(r)
        toks += r["tokens"]
    toks = toks[:M]
    dec.close()
    plain = la.LookaheadDecoder(cfg.with_(W=0, G=0), dev_w, 1024)
    ref = [plain.prefill(prompt)]
    dmax = 0.0
    while len(ref) < M:
        n = len(ref)
        ref += plain.step()["tokens"]
        if n in la_logits and toks[:n] == ref[:n]:
            dmax = max(dmax, float(np.max(np.abs(la_logits[n] - plain.debug_logits()[0]))))
    plain.close()
    div = next((i for i in range(M) if toks[i] != ref[i]), None)
    log(f"[7b] {len(steps)} lookahead steps; first divergence from plain decoding: {div}; "
        f"max |row-0 logit difference| before it {dmax:.3f}")
    # each run is within MAX_TOL of the exact logits
    assert dmax <= 2 * MAX_TOL
    if div is not None:  # 0: the two contexts' prefills (different launch shapes) part
        orc = oracle.Oracle(cfg, lasynth.host_bits(dev_w), len(prompt) + div + 8)
        _, lo = orc.extend([int(x) for x in prompt] + toks[:div], logits=True)
        z = lo[-1].astype(np.float32)
        gap = [float(z.max() - z[t]) for t in (toks[div], ref[div])]
        log(f"[7b] at the divergence the oracle ranks the two tokens {gap[0]:.3f} and "
            f"{gap[1]:.3f} below its best (top-2 margin {margin(lo[-1]):.3f})")
        assert max(gap) <= DECISION_MARGIN
