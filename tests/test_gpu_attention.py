"""One layer's masked attention kernel (la_attention) vs the oracle (GPU only).

Kernel-only workload: 32 heads x 128, prefix 1024, 121 query rows (W15 N5
G15), Q/K/V ~ N(0,1) in bf16.

Tolerance, from the kernel's arithmetic: the probabilities enter the PV
product as bf16 and the output is stored as bf16, each a round-to-nearest
with unit roundoff 2^-8 (bf16 keeps 8 significant bits), with fp32 sums
elsewhere.  For an output element o = sum_i p_i v_i / sum_i p_i the first
contributes at most 2^-8 * sum_i p_i |v_i| / sum_i p_i <= 2^-8 * max |v|
(over the head's values) and the second 2^-8 * |o|, so per element
    |got - ref| <= 2^-8 * (max |v| + |ref|) + 1e-4,
the last term for the fp32 accumulation.  Plus a relative Frobenius error
<= 1e-2 over the whole output.
"""
import numpy as np
import pytest
import torch

import lasynth
import lookahead_decoding_la_amd as la
import oracle
from lockstep import log

pytestmark = pytest.mark.gpu


BF16_NAN = 0x7FC0


def _run(a, past=0):
    """la_attention on the inputs of `a`, the cache rows padded to a multiple
    of 64 positions; the positions past the context hold the bf16 pattern
    `past` (0, or a NaN: the kernel must not let them reach the output)."""
    T, H, Hkv, dh, L = a["T"], a["n_heads"], a["n_kv_heads"], a["head_dim"], a["prefix"]
    ctx = ((L + T + 63) // 64) * 64
    dev = torch.device("cuda")
    q = torch.from_numpy(a["q"].view(np.int16)).to(dev)
    k = torch.full((Hkv, ctx, dh), past, dtype=torch.int16, device=dev)
    k[:, :L + T] = torch.from_numpy(a["k"].view(np.int16)).to(dev)
    vt = torch.full((Hkv, dh, ctx), past, dtype=torch.int16, device=dev)
    vt[:, :, :L + T] = torch.from_numpy(a["v"].view(np.int16)).to(dev).transpose(1, 2)
    out = torch.zeros((T, H, dh), dtype=torch.int16, device=dev)
    la.attention(q, k, vt.contiguous(), out, H, Hkv, L, a["W"], a["N"], a["G"])
    torch.cuda.synchronize()
    got = lasynth.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16)).astype(np.float64)
    cfg = lasynth.get_config("tiny", n_heads=H, n_kv_heads=Hkv, head_dim=dh,
                             W=a["W"], N=a["N"], G=a["G"])
    ref = oracle.attention(cfg, L, a["q"], a["k"], a["v"], bf16=True)
    vmax = np.abs(lasynth.bf16_bits_to_f32(a["v"])).max(axis=(1, 2))  # per KV head
    return got, ref, vmax[(np.arange(H) * Hkv) // H]  # per query head


CASES = [
    dict(),                                            # the kernel-only workload
    dict(prefix=0),                                    # block keys only
    dict(prefix=37, W=3, N=4, G=2),                    # ragged prefix, 16 rows
    dict(prefix=200, W=0, N=4, G=3),                   # 10 rows (padding)
    dict(prefix=130, n_heads=8, n_kv_heads=2),         # grouped KV heads
    dict(prefix=64, W=25, N=5, G=25),                  # 201 rows
    dict(prefix=5, W=1, N=2, G=0),                     # 2 rows
    dict(prefix=2000, n_heads=4, W=7, N=5, G=7),       # longer context, 57 rows (64-row group)
    dict(prefix=1100, n_heads=8, W=10, N=5, G=10),     # 81 rows: 3 row groups, last holds 17
    dict(prefix=300, n_heads=8, n_kv_heads=2, W=3, N=5, G=8),  # 45 rows, grouped KV heads
    dict(prefix=64, n_heads=4, W=4, N=5, G=4),         # 33 rows: a wave's second tile empty
    dict(prefix=700, n_heads=4, W=12, N=5, G=12),      # 97 rows: last group has one tile
    dict(prefix=1900, n_heads=8, W=10, N=5, G=10),     # 81 rows, cache rows of 1984 keys (per-tile kernel, 16 chunks)
    dict(prefix=2100, W=3, N=4, G=2),                  # 16 rows at 2100 committed keys: split kernel + merge
    dict(prefix=2100, n_heads=4, W=12, N=5, G=12),     # 97 rows above 2048 keys: split, 32-row groups
    dict(prefix=2100, n_heads=2, W=25, N=5, G=25),     # 201 rows above 2048 keys: split, one 128-row group per head
    dict(prefix=700, n_heads=256, n_kv_heads=32, W=3, N=3, G=3),  # 13 rows, 256 heads: per-tile kernel for a small block
    dict(prefix=0, W=0, N=2, G=0),                     # one row (plain decode), one key
    dict(prefix=13, n_heads=8, n_kv_heads=2, W=0, N=2, G=0),  # one row, 14 keys: one 32-key block, grouped KV heads
    dict(prefix=127, W=0, N=2, G=0),                   # one row, 128 keys: whole 32-key blocks, 2 key splits
    dict(prefix=2100, W=0, N=2, G=0),                  # one row, 2101 keys, 32 heads: 8 key splits + merge
    dict(prefix=1000, n_heads=256, n_kv_heads=32, W=0, N=2, G=0),  # one row, 256 heads: 2 key splits
    dict(prefix=300, n_heads=1024, n_kv_heads=128, W=0, N=2, G=0),  # one row, 1024 heads: the shallow-prefetch loop
]


# Cache rows whose positions past the context hold NaN (la_attention makes no
# assumption about them): the per-tile kernel, the split kernel and the row
# kernel, each with a last chunk or block that reaches past the context.
NAN_CASES = [
    dict(),                                            # per-tile kernel, 1145 keys in 1152
    dict(prefix=2100, W=3, N=4, G=2),                  # split kernel + merge
    dict(prefix=13, n_heads=8, n_kv_heads=2, W=0, N=2, G=0),  # row kernel, 14 keys
]


@pytest.mark.parametrize("kw", CASES, ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()) or "attn")
def test_attention_matches_oracle(kw):
    _check(kw, 0)


@pytest.mark.parametrize("kw", NAN_CASES, ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()) or "attn")
def test_attention_ignores_nan_past_the_context(kw):
    _check(kw, BF16_NAN)


def _check(kw, past):
    a = lasynth.make_attn_inputs(seed=7, **kw)
    log(f"[attention] {kw} T={a['T']} past-context fill {past:#06x}")
    got, ref, vmax = _run(a, past)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    bound = 2.0**-8 * (vmax[None, :, None] + np.abs(ref)) + 1e-4
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    log(f"  max={err.max():.3e} (worst fraction of the bound {np.max(err / bound):.2f}) rel={rel:.3e}")
    assert np.all(err <= bound)
    assert rel <= 1e-2
