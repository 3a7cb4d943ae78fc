"""Pipelined stepping (la_step_submit / la_step_collect): with two steps in
flight every collected result equals what la_step returns for the same
step, and the context refuses other calls while steps are in flight.

GPU tests: a bf16 context (the 7B-step kernels at a small width) and an
fp32 tiny one, each stepped by la_step and, from the same prefill, by the
pipelined pair; the results (tokens, accepted count, winner, KV length)
must be identical, since both run the same kernels on the same state."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import lasynth  # noqa: E402
import lookahead_decoding_la_amd as la  # noqa: E402

pytestmark = pytest.mark.gpu

CONFIGS = [
    lasynth.get_config("tiny"),
    lasynth.get_config("7b", name="bf16_w15_small", n_layers=3, d_model=512, n_heads=4,
                       n_kv_heads=4, d_ffn=1408, vocab=2048, prompt_len=64, span_len=8, n_spans=2),
]


def _decoder(cfg, dev_w):
    d = la.LookaheadDecoder(cfg, dev_w, 512)
    p = lasynth.make_prompt(cfg)
    d.prefill(p, lasynth.make_init_window(cfg, p) if cfg.W else None)
    return d


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_pipelined_equals_step(cfg):
    dev_w = la.upload_weights(lasynth.make_weights(cfg))
    steps = 12
    ref = _decoder(cfg, dev_w)
    want = [ref.step() for _ in range(steps)]
    pipe = _decoder(cfg, dev_w)
    got = []
    pipe.step_submit()
    for i in range(steps):
        if i + 1 < steps:
            pipe.step_submit()  # two in flight
        got.append(pipe.step_collect())
    assert got == want
    # after the pipeline drains the context steps normally again
    assert pipe.step() == ref.step()


def test_pipelined_state_errors():
    cfg = lasynth.get_config("tiny")
    d = _decoder(cfg, la.upload_weights(lasynth.make_weights(cfg)))
    with pytest.raises(la.LaError) as e:
        d.step_collect()  # nothing in flight
    assert e.value.status == la.LA_ERR_STATE
    d.step_submit()
    d.step_submit()
    for call in (d.step_submit, d.step, d.debug_state):
        with pytest.raises(la.LaError) as e:
            call()
        assert e.value.status == la.LA_ERR_STATE
    d.step_collect()
    d.step_collect()
    d.step()


def test_pipelined_batch_equals_step():
    # two sequences per forward pass, each with its own prompt: every collected
    # result list (one result per sequence) equals la_step's
    cfg = lasynth.get_config("tiny")
    dev_w = la.upload_weights(lasynth.make_weights(cfg))
    p0 = lasynth.make_prompt(cfg)
    p1 = lasynth.make_prompt(cfg, seed=1)

    def make():
        d = la.LookaheadDecoder(cfg, dev_w, 512, batch=2)
        for s, p in enumerate((p0, p1)):
            d.prefill(p, lasynth.make_init_window(cfg, p), seq=s)
        return d

    ref, pipe = make(), make()
    want = [ref.step() for _ in range(8)]
    got = []
    pipe.step_submit()
    for i in range(8):
        if i + 1 < 8:
            pipe.step_submit()
        got.append(pipe.step_collect())
    assert got == want


def test_submit_reserves_capacity_for_steps_in_flight():
    """A submit assumes each step in flight commits its maximum of N
    tokens: with room for one step only (prompt + step rows + N - 1 tokens
    of capacity) the first submit is accepted and the second refused with
    LA_ERR_OUT_OF_CAPACITY (a host-side check: nothing is launched), and
    the context keeps working: the step in flight collects normally."""
    cfg = lasynth.get_config("tiny")
    p = lasynth.make_prompt(cfg)
    cap = len(p) + cfg.T + cfg.N - 1
    d = la.LookaheadDecoder(cfg, la.upload_weights(lasynth.make_weights(cfg)), cap)
    d.prefill(p, lasynth.make_init_window(cfg, p))
    d.step_submit()
    with pytest.raises(la.LaError) as e:
        d.step_submit()
    assert e.value.status == la.LA_ERR_OUT_OF_CAPACITY
    r = d.step_collect()
    assert 1 <= r["n_emitted"] <= cfg.N and r["kv_len"] == len(p) + r["n_emitted"]
    kv, _ = d.debug_state()
    assert kv == r["kv_len"]
