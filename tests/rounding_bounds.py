"""Derive the full-depth logit tolerances of the bf16 datapath (GPU, fp64).

    python tests/rounding_bounds.py [--out PATH] [7b 13b 34b]
        (default PATH: tests/golden/rounding_bounds.json)

A bf16 datapath stores activations as bf16 at seven points of each layer
and accumulates everything else in fp32.  This script measures how far that
storage alone moves the logits, on the same seeded weights the full-size
tests draw (lasynth.make_weights_device) and the first TOKENS tokens of the
workload's prompt (causal forward): one forward in fp64 with no rounding,
one in fp64 that rounds to bf16 (torch's conversion: through fp32, nearest
even) at all seven points, and one per point with only that point rounded:

  1. the GEMM input of the attention block, x * w_attn_norm (the 1/rms
     factor is applied to the products afterwards);
  2. q and k after the rotary embedding, and v (the query buffer and the
     KV cache);
  3. the attention probabilities exp(s - max) entering the PV product (the
     normaliser sums the unrounded values);
  4. the attention output (input of the O projection);
  5. the GEMM input of the FFN block, x * w_ffn_norm (1/rms afterwards);
  6. the SwiGLU output (input of the down projection);
  7. the LM-head input, RMSNorm(x) * w_final_norm.

These are the storage points of the oracle's bf16 storage mode.  The
residual stream stays unrounded.  Recorded per shape: the largest and rms
|logit difference| over all rows and the vocabulary with all seven points
("max_abs_dlogit", "rms_dlogit"), and the same for each point alone
("by_point").  Tests take 1.5x max_abs_dlogit as the bound of one bf16 run
against exact arithmetic.

This is test infrastructure: torch only, no call into the HIP library.
"""
import json
import math
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
import lasynth  # noqa: E402

TOKENS = 32
OUT = os.path.join(HERE, "golden", "rounding_bounds.json")


def bf(x):
    return x.to(torch.bfloat16).to(x.dtype)


VARIANTS = ["exact", "all"] + [f"only_{k}" for k in range(1, 8)]


def _rounders(variant):
    """r[k](v): point k's storage for this variant (bf16 or identity)."""
    ident = lambda v: v
    if variant == "exact":
        on = set()
    elif variant == "all":
        on = set(range(1, 8))
    else:
        on = {int(variant.split("_")[1])}
    return {k: (bf if k in on else ident) for k in range(1, 8)}


def measure(name):
    cfg = lasynth.get_config(name)
    dev = torch.device("cuda")
    W = lasynth.make_weights_device(cfg, seed=0)
    names = [n for n, _ in lasynth.weight_shapes(cfg)]
    wt = dict(zip(names, W))
    f64 = lambda n: wt[n].to(torch.float64)
    d, H, Hkv, dh = cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    T = TOKENS
    toks = torch.as_tensor(lasynth.make_prompt(cfg)[:T].astype("int64"), device=dev)
    pos = torch.arange(T, dtype=torch.float64, device=dev)
    inv = cfg.rope_theta ** (-torch.arange(0, dh, 2, dtype=torch.float64, device=dev) / dh)
    ang = pos[:, None] * inv[None]
    cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
    mask = torch.triu(torch.full((T, T), -math.inf, dtype=torch.float64, device=dev), 1)

    def rope(x):  # adjacent pairs (2i, 2i+1)
        a, b = x[..., 0::2], x[..., 1::2]
        o = torch.empty_like(x)
        o[..., 0::2] = a * cos - b * sin
        o[..., 1::2] = a * sin + b * cos
        return o

    def inv_rms(x):
        return 1.0 / torch.sqrt((x * x).mean(-1, keepdim=True) + cfg.rms_eps)

    emb = f64("tok_emb")[toks]
    rs = {v: _rounders(v) for v in VARIANTS}
    xs = {v: emb.clone() for v in VARIANTS}
    for l in range(cfg.n_layers):
        p = f"l{l}."
        wq, wk, wv, wo = f64(p + "wq"), f64(p + "wk"), f64(p + "wv"), f64(p + "wo")
        for var in VARIANTS:
            r, x = rs[var], xs[var]
            a = r[1](x * f64(p + "attn_norm"))
            s = inv_rms(x)
            q = r[2](rope(((a @ wq.T) * s).view(T, H, dh)))
            k = r[2](rope(((a @ wk.T) * s).view(T, Hkv, dh)))
            v = r[2](((a @ wv.T) * s).view(T, Hkv, dh))
            k = k.repeat_interleave(H // Hkv, dim=1)
            v = v.repeat_interleave(H // Hkv, dim=1)
            qh = q.permute(1, 0, 2).contiguous()  # [H][T][dh]
            kh = k.permute(1, 2, 0).contiguous()  # [H][dh][T]
            vh = v.permute(1, 0, 2).contiguous()  # [H][T][dh]
            sc = torch.matmul(qh, kh) / math.sqrt(dh) + mask
            e = torch.exp(sc - sc.amax(-1, keepdim=True))
            o = torch.matmul(r[3](e), vh) / e.sum(-1, keepdim=True)  # [H][T][dh]
            xs[var] = x + r[4](o.permute(1, 0, 2).reshape(T, H * dh)) @ wo.T
        del wq, wk, wv, wo
        wg, wu, wd = f64(p + "w_gate"), f64(p + "w_up"), f64(p + "w_down")
        for var in VARIANTS:
            r, x = rs[var], xs[var]
            a = r[5](x * f64(p + "ffn_norm"))
            s = inv_rms(x)
            g, u = (a @ wg.T) * s, (a @ wu.T) * s
            xs[var] = x + r[6](torch.nn.functional.silu(g) * u) @ wd.T
        del wg, wu, wd
    lm = f64("lm_head")
    lg = {}
    for var in VARIANTS:
        x = xs[var]
        lg[var] = rs[var][7](x * inv_rms(x) * f64("final_norm")) @ lm.T

    def stats(var):
        dd = (lg[var] - lg["exact"]).abs()
        return {"max_abs_dlogit": float(dd.max()), "rms_dlogit": float(dd.pow(2).mean().sqrt())}

    res = {"layers": cfg.n_layers, "d_model": d, "tokens": T, **stats("all"),
           "logit_std": float(lg["exact"].std()),
           "by_point": {v: stats(v) for v in VARIANTS[2:]}}
    print(name, json.dumps(res), flush=True)
    del W, wt
    torch.cuda.empty_cache()
    return res


def main():
    args = sys.argv[1:]
    path = OUT
    if "--out" in args:
        i = args.index("--out")
        path = args[i + 1]
        del args[i:i + 2]
    names = args or ["7b", "13b", "34b"]
    out = json.load(open(path)) if os.path.exists(path) else {}
    for n in names:
        out[n] = measure(n)
        json.dump(out, open(path, "w"), indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
