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
