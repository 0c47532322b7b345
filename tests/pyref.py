"""Pure-Python, loop-by-loop reference pieces used to pin the oracle on tiny inputs.

They are written from the definitions independently of the oracle's vectorised numpy code:
no numpy, explicit loops, math.exp. Only usable for a few dozen tokens.
"""
import math


def scores(q, k, scale):
    """S[r][c] = scale * sum_d q[r][d] k[c][d] as nested Python lists."""
    n, d = len(q), len(q[0])
    return [[scale * sum(q[r][e] * k[c][e] for e in range(d)) for c in range(n)] for r in range(n)]


def masked_attention(q, k, v, allowed_cols_per_row, scale):
    """out[r] = softmax over allowed columns of S[r] applied to v; zero row if none allowed."""
    s = scores(q, k, scale)
    n, dv = len(q), len(v[0])
    out = []
    for r in range(n):
        cols = [c for c in range(n) if allowed_cols_per_row[r][c]]
        if not cols:
            out.append([0.0] * dv)
            continue
        mx = max(s[r][c] for c in cols)
        w = {c: math.exp(s[r][c] - mx) for c in cols}
        z = sum(w.values())
        out.append([sum(w[c] * v[c][e] for c in cols) / z for e in range(dv)])
    return out


def brute_flags(q, k, skipped, tile_q, tile_k, scale, log_eps, descending, dense_prefix=0):
    """Flags and margins per (row tile, key tile) computed from scratch for every tile:
    the running maximum of a row before tile j is recomputed as the maximum over all columns
    of all tiles visited earlier in this step (no incremental state)."""
    n = len(q)
    s = scores(q, k, scale)
    tq = -(-n // tile_q)
    tk = -(-n // tile_k)
    flags = [[False] * tk for _ in range(tq)]
    margins = [[None] * tk for _ in range(tq)]
    for i in range(tq):
        rows = list(range(i * tile_q, min(n, (i + 1) * tile_q)))
        seq = list(range(tk))
        if descending:
            seq.reverse()
        visited = [j for j in seq if not skipped[i][j]]
        for pos, j in enumerate(visited):
            before = visited[:pos]
            cols_j = range(j * tile_k, min(n, (j + 1) * tile_k))
            worst = -math.inf
            for r in rows:
                local = max(s[r][c] for c in cols_j)
                if before:
                    prev = max(s[r][c] for jj in before
                               for c in range(jj * tile_k, min(n, (jj + 1) * tile_k)))
                    diff = local - prev
                else:
                    diff = math.inf
                worst = max(worst, diff)
            margin = worst - log_eps
            margins[i][j] = margin
            exempt = (i * tile_q < dense_prefix) or (j * tile_k < dense_prefix)
            flags[i][j] = (margin < 0) and not exempt
    return flags, margins
