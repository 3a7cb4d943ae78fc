"""Derive the full-depth logit tolerances of the bf16 datapath (GPU, fp64).

    python tests/rounding_bounds.py [--out PATH] [7b 13b 34b]
        (default PATH: tests/golden/rounding_bounds.json)

The bf16 library stores activations as bf16 at seven points of each layer
and accumulates everything else in fp32.  This script measures how far that
storage alone moves the logits, on the same seeded weights the full-size
tests draw (lasynth.make_weights_device) and the first TOKENS tokens of the
workload's prompt (causal forward): one forward in fp64 with no rounding,
one in fp64 that rounds to bf16 (nearest even) exactly where the library
stores bf16:

  1. the GEMM input of the attention block, x * w_attn_norm (the 1/rms
     factor is applied to the fp32 product afterwards);
  2. q and k after the rotary embedding, and v (the query buffer and the
     KV cache);
  3. the attention probabilities exp(s - max) entering the PV product (the
     normaliser sums the unrounded values);
  4. the attention output (input of the O projection);
  5. the GEMM input of the FFN block, x * w_ffn_norm (1/rms afterwards);
  6. the SwiGLU output (input of the down projection);
  7. the LM-head input, x * w_final_norm (1/rms afterwards).

The residual stream stays fp32 in the library and unrounded here.  The
recorded figure per shape is the largest |logit difference| over all rows
and the vocabulary; tests take 1.5x it as the bound of one bf16 run against
exact arithmetic, and twice that for two bf16 runs against each other (each
is within the bound of the exact logits).

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
    xs = [emb.clone(), emb.clone()]  # exact, rounded
    for l in range(cfg.n_layers):
        p = f"l{l}."
        wq, wk, wv, wo = f64(p + "wq"), f64(p + "wk"), f64(p + "wv"), f64(p + "wo")
        for i, rnd in enumerate((False, True)):
            r = bf if rnd else (lambda v: v)
            x = xs[i]
            a = r(x * f64(p + "attn_norm"))
            s = inv_rms(x)
            q = r(rope(((a @ wq.T) * s).view(T, H, dh)))
            k = r(rope(((a @ wk.T) * s).view(T, Hkv, dh)))
            v = r(((a @ wv.T) * s).view(T, Hkv, dh))
            k = k.repeat_interleave(H // Hkv, dim=1)
            v = v.repeat_interleave(H // Hkv, dim=1)
            qh = q.permute(1, 0, 2).contiguous()  # [H][T][dh]
            kh = k.permute(1, 2, 0).contiguous()  # [H][dh][T]
            vh = v.permute(1, 0, 2).contiguous()  # [H][T][dh]
            sc = torch.matmul(qh, kh) / math.sqrt(dh) + mask
            e = torch.exp(sc - sc.amax(-1, keepdim=True))
            o = torch.matmul(r(e), vh) / e.sum(-1, keepdim=True)  # [H][T][dh]
            x = x + r(o.permute(1, 0, 2).reshape(T, H * dh)) @ wo.T
            xs[i] = x
        del wq, wk, wv, wo
        wg, wu, wd = f64(p + "w_gate"), f64(p + "w_up"), f64(p + "w_down")
        for i, rnd in enumerate((False, True)):
            r = bf if rnd else (lambda v: v)
            x = xs[i]
            a = r(x * f64(p + "ffn_norm"))
            s = inv_rms(x)
            g, u = (a @ wg.T) * s, (a @ wu.T) * s
            xs[i] = x + r(torch.nn.functional.silu(g) * u) @ wd.T
        del wg, wu, wd
    lm = f64("lm_head")
    lg = []
    for i, rnd in enumerate((False, True)):
        r = bf if rnd else (lambda v: v)
        x = xs[i]
        lg.append((r(x * f64("final_norm")) @ lm.T) * inv_rms(x))
    dd = (lg[1] - lg[0]).abs()
    res = {"layers": cfg.n_layers, "d_model": d, "tokens": T,
           "max_abs_dlogit": float(dd.max()),
           "rms_dlogit": float(dd.pow(2).mean().sqrt()),
           "logit_std": float(lg[0].std())}
    print(name, res, flush=True)
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
