"""One layer's masked attention kernel (la_attention) vs the oracle (GPU only).

Kernel-only workload: 32 heads x 128, prefix 1024, 121 query rows (W15 N5
G15), Q/K/V ~ N(0,1) in bf16.  Tolerance: max |diff| <= 1e-2 and relative
Frobenius error <= 1e-2 (bf16 output rounding is 2^-9 relative).
"""
import numpy as np
import pytest
import torch

import lasynth
import lookahead_decoding_la_amd as la
import oracle
from lockstep import log

pytestmark = pytest.mark.gpu


def _run(a):
    T, H, Hkv, dh, L = a["T"], a["n_heads"], a["n_kv_heads"], a["head_dim"], a["prefix"]
    ctx = ((L + T + 63) // 64) * 64
    dev = torch.device("cuda")
    q = torch.from_numpy(a["q"].view(np.int16)).to(dev)
    k = torch.zeros((Hkv, ctx, dh), dtype=torch.int16, device=dev)
    k[:, :L + T] = torch.from_numpy(a["k"].view(np.int16)).to(dev)
    vt = torch.zeros((Hkv, dh, ctx), dtype=torch.int16, device=dev)
    vt[:, :, :L + T] = torch.from_numpy(a["v"].view(np.int16)).to(dev).transpose(1, 2)
    out = torch.zeros((T, H, dh), dtype=torch.int16, device=dev)
    la.attention(q, k, vt.contiguous(), out, H, Hkv, L, a["W"], a["N"], a["G"])
    torch.cuda.synchronize()
    got = lasynth.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16)).astype(np.float64)
    cfg = lasynth.get_config("tiny", n_heads=H, n_kv_heads=Hkv, head_dim=dh,
                             W=a["W"], N=a["N"], G=a["G"])
    ref = oracle.attention(cfg, L, a["q"], a["k"], a["v"], bf16=True)
    return got, ref


CASES = [
    dict(),                                            # the kernel-only workload
    dict(prefix=0),                                    # block keys only
    dict(prefix=37, W=3, N=4, G=2),                    # ragged prefix, 16 rows
    dict(prefix=200, W=0, N=4, G=3),                   # 10 rows (padding)
    dict(prefix=130, n_heads=8, n_kv_heads=2),         # grouped KV heads
    dict(prefix=64, W=25, N=5, G=25),                  # 201 rows
    dict(prefix=5, W=1, N=2, G=0),                     # 2 rows
    dict(prefix=2000, n_heads=4, W=7, N=5, G=7),       # longer context
]


@pytest.mark.parametrize("kw", CASES, ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()) or "attn")
def test_attention_matches_oracle(kw):
    a = lasynth.make_attn_inputs(seed=7, **kw)
    log(f"[attention] {kw} T={a['T']}")
    got, ref = _run(a)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    log(f"  max={err.max():.3e} rel={rel:.3e}")
    assert err.max() <= 1e-2
    assert rel <= 1e-2
