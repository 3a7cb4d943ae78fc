"""Test-side helpers (no method arithmetic beyond what a test states)."""


def trajectory_rows(W, N, G, r):
    """Block rows that row r reads, in position order, written from the 2D
    window's description: lookahead row (l, j) reads the current token, the
    level-1 entries of columns 0..j, then entries of its own column at levels
    2..l; candidate row (g, i) reads the current token and the first i tokens
    of candidate g; the current token reads only itself."""
    n1 = N - 1

    def la(l, j):
        return 1 + (l - 1) * W + j

    def cd(g, i):
        return 1 + n1 * W + g * n1 + (i - 1)

    if r == 0:
        return [0]
    if r <= n1 * W:
        l, j = 1 + (r - 1) // W, (r - 1) % W
        return [0] + [la(1, jj) for jj in range(j + 1)] + \
            [la(ll, j) for ll in range(2, l + 1)]
    g, i = (r - 1 - n1 * W) // n1, 1 + (r - 1 - n1 * W) % n1
    return [0] + [cd(g, ii) for ii in range(1, i + 1)]


def definition_probs(z, T, k, p):
    """Probability of each token under the draw's definition, from its
    description: tokens ordered by logit (fp32), descending, lower id first
    on ties; the first k kept (all for k = 0); weights exp((z - z_max) / T);
    the shortest prefix holding a fraction p of the weight kept; weights
    renormalized over what is kept."""
    import numpy as np
    z = np.asarray(z, np.float32).astype(np.float64)
    order = sorted(range(z.size), key=lambda j: (-z[j], j))
    n = k if 0 < k < z.size else z.size
    kept = order[:n]
    w = np.exp((z[kept] - z[kept[0]]) / T)
    if p < 1.0:
        c = np.cumsum(w)
        m = int(np.argmax(c >= p * c[-1])) + 1
        kept, w = kept[:m], w[:m]
    out = np.zeros(z.size)
    out[kept] = w / w.sum()
    return out


def rounding_record(name):
    """The rounding-only record of workload `name` (tests/rounding_bounds.py,
    stored in tests/golden/rounding_bounds.json): how far storing the seven
    bf16 activations alone moves the logits from exact arithmetic, on the
    same weights (max and rms |logit difference|)."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "rounding_bounds.json")
    with open(path) as f:
        return json.load(f)[name]


def full_depth_bounds(name):
    """Bounds of one full-depth bf16 run of workload `name` against the
    exact oracle, from its rounding-only record (max m, rms s):
      - every logit within 1.5 m;
      - the rms logit difference within 1.5 s;
      - a decision may differ from the oracle's only where the oracle's
        top-2 margin is at most 5 sqrt(2) s: the logits' errors act on a
        decision through the gap between two of them, whose error has about
        sqrt(2) s standard deviation, and a gap error beyond five of those
        is not expected in any run these tests make (about 1e-6 per
        decision for a normal error)."""
    r = rounding_record(name)
    m, s = r["max_abs_dlogit"], r["rms_dlogit"]
    return 1.5 * m, 1.5 * s, 5.0 * 2 ** 0.5 * s


def full_depth_logit_tol(name):
    """The per-logit bound of full_depth_bounds (1.5x the rounding-only max)."""
    return full_depth_bounds(name)[0]
