"""Pin the oracle's one-layer masked attention (kernel-only workload) to torch
scaled_dot_product_attention over each row's key sequence: the whole prefix
followed by the block rows on the row's window trajectory."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import lasynth
import oracle
from helpers import trajectory_rows


def _ref(cfg, L, q, k, v, valid):
    T, H, dh = q.shape
    Hkv = k.shape[0]
    out = np.zeros((T, H, dh))
    for r in range(T):
        if not valid[r]:
            continue
        rows = trajectory_rows(cfg.W, cfg.N, cfg.G, r)
        assert all(valid[s] for s in rows)
        keys = list(range(L)) + [L + s for s in rows]
        for h in range(H):
            kh = h * Hkv // H
            qq = torch.from_numpy(q[r, h][None, None, None, :])
            kk = torch.from_numpy(k[kh, keys][None, None])
            vv = torch.from_numpy(v[kh, keys][None, None])
            out[r, h] = F.scaled_dot_product_attention(qq, kk, vv)[0, 0, 0].numpy()
    return out


@pytest.mark.parametrize("H,Hkv,dh,L,W,N,G,nvalid", [
    (4, 2, 16, 20, 3, 4, 2, 2),
    (2, 2, 32, 0, 4, 3, 3, 1),
    (4, 1, 8, 7, 2, 2, 4, 0),
    (3, 3, 16, 33, 0, 5, 2, 2),
])
def test_attention_matches_sdpa(H, Hkv, dh, L, W, N, G, nvalid):
    cfg = lasynth.get_config("tiny", n_heads=H, n_kv_heads=Hkv, head_dim=dh,
                             W=W, N=N, G=G)
    T = cfg.T
    rng = np.random.default_rng(H * 1000 + L)
    q = rng.standard_normal((T, H, dh)).astype(np.float32)
    k = rng.standard_normal((Hkv, L + T, dh)).astype(np.float32)
    v = rng.standard_normal((Hkv, L + T, dh)).astype(np.float32)
    valid = np.ones(T, np.int32)
    n1 = N - 1
    for g in range(nvalid, G):
        valid[1 + n1 * W + g * n1: 1 + n1 * W + (g + 1) * n1] = 0
    got = oracle.attention(cfg, L, q, k, v, bf16=False, valid=valid)
    ref = _ref(cfg, L, q.astype(np.float64), k.astype(np.float64),
               v.astype(np.float64), valid)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_bf16_inputs_widen_exactly():
    a = lasynth.make_attn_inputs(seed=1, n_heads=2, head_dim=16, prefix=9,
                                 W=2, N=3, G=2)
    cfg = lasynth.get_config("tiny", n_heads=2, n_kv_heads=2, head_dim=16,
                             W=2, N=3, G=2)
    got = oracle.attention(cfg, 9, a["q"], a["k"], a["v"], bf16=True)
    f = lambda x: lasynth.bf16_bits_to_f32(x).astype(np.float64)
    ref = _ref(cfg, 9, f(a["q"]), f(a["k"]), f(a["v"]), np.ones(cfg.T, np.int32))
    assert np.max(np.abs(got - ref)) < 1e-12
