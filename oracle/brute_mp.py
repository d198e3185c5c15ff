"""Brute-force scaled dot-product attention in 50-digit arithmetic (mpmath).

TEST INFRASTRUCTURE ONLY (same rule as ``sdpa_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may use it).

A second, separately written evaluation of Eq. (1) of 《精读 Attention Is All
You Need：原始 Transformer 论文》 ("缩放点积注意力：点积为什么要缩放"), with
scalar loops only and no array library, used to check the fp64 oracle on tiny
shapes.  For every query i it walks the keys j, keeps those that are legal
(causal: j ≤ i, per 《Attention Is All You Need：注意力就是你所需要的一切》
§3.2.3; padding: j < clamp(len, 0, m)), forms exp(scale · q_i·k_j) over them
only (illegal keys carry weight exactly zero), and divides the weighted sum of
the values by the sum of the exponentials.  A query with no legal key yields
the zero vector.  It does not subtract a row maximum: at 50 digits and the
small magnitudes used in tests nothing overflows, which makes this a genuinely
different route from the oracle's.
"""

from __future__ import annotations

import mpmath


def attention_mp(q, k, v, scale, causal=False, key_lens=None, dps=50, window=None, keep=None,
                 keep_scale=1.0):
    """q: [B][h][n][d_k], k: [B][h][m][d_k], v: [B][h][m][d_v] nested sequences.

    ``window``: None or (left, right, align): key j is legal for query i only
    if p − left ≤ j ≤ p + right, where p = i (align 'top_left') or
    p = i + len − n (align 'bottom_right': the queries end where the keys end);
    a None side is unbounded.

    ``keep`` (attention dropout): None, or [B][h][n][m] booleans; a legal key
    then still counts in the denominator, but its value enters the sum only if
    kept, and the sum is multiplied by ``keep_scale``.

    Returns nested lists of ``mpmath.mpf`` with shape [B][h][n][d_v].
    """
    with mpmath.workdps(dps):
        sc = mpmath.mpf(scale) if not isinstance(scale, mpmath.mpf) else scale
        out = []
        for b in range(len(q)):
            L = None if key_lens is None else int(key_lens[b])
            heads = []
            for hh in range(len(q[b])):
                Q, K, V = q[b][hh], k[b][hh], v[b][hh]
                m = len(K)
                d_v = len(V[0]) if m else 0
                lim = m if L is None else min(max(L, 0), m)
                rows = []
                for i in range(len(Q)):
                    num = [mpmath.mpf(0)] * d_v
                    den = mpmath.mpf(0)
                    if window is not None:
                        p = i if window[2] == "top_left" else i + lim - len(Q)
                    for j in range(m):
                        if j >= lim or (causal and j > i):
                            continue
                        if window is not None:
                            if window[0] is not None and j < p - window[0]:
                                continue
                            if window[1] is not None and j > p + window[1]:
                                continue
                        dot = mpmath.fsum(mpmath.mpf(float(Q[i][t])) * mpmath.mpf(float(K[j][t]))
                                          for t in range(len(Q[i])))
                        e = mpmath.exp(sc * dot)
                        den += e
                        if keep is not None and not keep[b][hh][i][j]:
                            continue
                        for c in range(d_v):
                            num[c] += e * mpmath.mpf(float(V[j][c]))
                    if den == 0:
                        rows.append([mpmath.mpf(0)] * d_v)
                    else:
                        ks = mpmath.mpf(1) if keep is None else mpmath.mpf(keep_scale)
                        rows.append([x / den * ks for x in num])
                heads.append(rows)
            out.append(heads)
        return out


def multihead_mp(xq, xkv, wq, wk, wv, wo, scale, causal=False, key_lens=None, dps=50):
    """The multi-head sublayer with scalar loops at ``dps`` digits: every
    projection is written out as sums of products, each head goes through
    ``attention_mp``, and the concatenated heads are multiplied by W^O.
    Shapes as in the oracle's ``multihead``.  Returns nested lists [B][n][d_model]."""
    with mpmath.workdps(dps):
        B, n, m = len(xq), len(xq[0]), len(xkv[0])
        h, d_model, d_k = len(wq), len(wq[0]), len(wq[0][0])
        d_v = len(wv[0][0])

        def proj(x, w, rows, width):
            # [b][head][row][col] = Σ_t x[b][row][t] · w[head][t][col]
            out = []
            for b in range(B):
                per_head = []
                for i in range(h):
                    per_head.append([[mpmath.fsum(mpmath.mpf(float(x[b][r][t])) *
                                                  mpmath.mpf(float(w[i][t][c]))
                                                  for t in range(d_model))
                                      for c in range(width)] for r in range(rows)])
                out.append(per_head)
            return out

        q = proj(xq, wq, n, d_k)
        k = proj(xkv, wk, m, d_k)
        v = proj(xkv, wv, m, d_v)
        heads = attention_mp(q, k, v, scale, causal=causal, key_lens=key_lens, dps=dps)
        out = []
        for b in range(B):
            rows = []
            for r in range(n):
                cat = [heads[b][i][r][c] for i in range(h) for c in range(d_v)]
                rows.append([mpmath.fsum(cat[t] * mpmath.mpf(float(wo[t][c])) for t in range(h * d_v))
                             for c in range(d_model)])
            out.append(rows)
        return out


def _legal_mp(i, j, n, m, causal, L, window):
    lim = m if L is None else min(max(L, 0), m)
    if j >= lim or (causal and j > i):
        return False
    if window is not None:
        p = i if window[2] == "top_left" else i + lim - n
        if window[0] is not None and j < p - window[0]:
            return False
        if window[1] is not None and j > p + window[1]:
            return False
    return True


def _head_loss_mp(Q, K, V, dO, sc, legal, keep=None, ks=None):
    """Σ_i dO_i · o_i for one head, every argument already ``mpf``; with
    ``keep`` the dropped weights leave the sum (not the denominator) and the
    sum is scaled by ``ks``."""
    total = mpmath.mpf(0)
    for i in range(len(Q)):
        den = mpmath.mpf(0)
        num = [mpmath.mpf(0)] * len(V[0])
        for j in range(len(K)):
            if not legal[i][j]:
                continue
            e = mpmath.exp(sc * mpmath.fsum(a * b for a, b in zip(Q[i], K[j])))
            den += e
            if keep is not None and not keep[i][j]:
                continue
            for c in range(len(num)):
                num[c] += e * V[j][c]
        if den != 0:
            mul = mpmath.mpf(1) if keep is None else ks
            total += mpmath.fsum(dO[i][c] * num[c] / den * mul for c in range(len(num)))
    return total


def attention_grad_fd_mp(q, k, v, do, scale, causal=False, key_lens=None, window=None, dps=60,
                         eps=1e-20, keep=None, keep_scale=1.0):
    """Gradients of ℓ = Σ dO ∘ Attention(Q, K, V) by central differences at
    ``dps`` digits, one input element at a time: (ℓ(x + ε) − ℓ(x − ε)) / 2ε.

    This is the derivative itself, not a formula for it: it evaluates Eq. (1)
    (legal keys only, no maximum subtraction, as ``attention_mp``) twice per
    element.  With ε = 1e-20 at 60 digits the truncation error is O(ε²) and
    the rounding error about 10^(−60)/ε, so the result is exact far beyond
    fp64.  ``keep``/``keep_scale``: attention dropout as in ``attention_mp``.
    Returns (dq, dk, dv) as nested lists of floats, shapes as q, k, v.
    """
    with mpmath.workdps(dps):
        sc = mpmath.mpf(scale)
        ep = mpmath.mpf(eps)
        ksc = mpmath.mpf(keep_scale)
        grads = ([], [], [])
        for b in range(len(q)):
            L = None if key_lens is None else int(key_lens[b])
            g_b = ([], [], [])
            for hh in range(len(q[b])):
                X = [[[mpmath.mpf(float(x)) for x in row] for row in t[b][hh]] for t in (q, k, v)]
                dO = [[mpmath.mpf(float(x)) for x in row] for row in do[b][hh]]
                n, m = len(X[0]), len(X[1])
                legal = [[_legal_mp(i, j, n, m, causal, L, window) for j in range(m)]
                         for i in range(n)]
                for which in range(3):
                    g = []
                    for r in range(len(X[which])):
                        row = []
                        for c in range(len(X[which][r])):
                            x0 = X[which][r][c]
                            X[which][r][c] = x0 + ep
                            kp = None if keep is None else keep[b][hh]
                            up = _head_loss_mp(X[0], X[1], X[2], dO, sc, legal, kp, ksc)
                            X[which][r][c] = x0 - ep
                            dn = _head_loss_mp(X[0], X[1], X[2], dO, sc, legal, kp, ksc)
                            X[which][r][c] = x0
                            row.append(float((up - dn) / (2 * ep)))
                        g.append(row)
                    g_b[which].append(g)
            for which in range(3):
                grads[which].append(g_b[which])
        return grads
