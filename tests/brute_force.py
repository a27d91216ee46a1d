"""Scalar-loop brute force of the routed attention, for tiny inputs (N <= 256).

Written independently of ``oracle/`` (no numpy vectorisation, no shared
helpers): plain Python floats and explicit loops over tokens, blocks and
dimensions.  Used only to pin the oracle.

Top-k selection here repeatedly takes the best remaining eligible block
(highest score, then lowest index) instead of sorting, so it checks the
oracle's sort-based top-k with a different algorithm.
"""

from __future__ import annotations

import math


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def brute_forward(q, k, v, *, block, causal, approx, mode, alpha=0.5, density=0.15, scale=None):
    """q: nested list [B][Hq][N][d]; k, v: [B][Hkv][N][d].  Returns (mask, out) with
    mask[b][h][I] a sorted list of selected blocks and out [B][Hq][N][d]."""
    B, Hq, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    M = (N + block - 1) // block
    start = [J * block for J in range(M)]
    stop = [min(N, (J + 1) * block) for J in range(M)]

    def mean_block(x, J):
        acc = [0.0] * d
        for t in range(start[J], stop[J]):
            for c in range(d):
                acc[c] += x[t][c]
        n = stop[J] - start[J]
        return [a / n for a in acc]

    def sum_block(x, J):
        acc = [0.0] * d
        for t in range(start[J], stop[J]):
            for c in range(d):
                acc[c] += x[t][c]
        return acc

    masks, outs = [], []
    for b in range(B):
        mb, ob = [], []
        for h in range(Hq):
            g = h // G
            kbar = [mean_block(k[b][g], J) for J in range(M)]
            vsum = [sum_block(v[b][g], J) for J in range(M)]
            mh, oh = [], [[0.0] * d for _ in range(N)]
            for I in range(M):
                qbar = mean_block(q[b][h], I)
                elig = [J for J in range(M) if (not causal) or J <= I]
                sc = {J: scale * _dot(qbar, kbar[J]) for J in elig}
                if mode == "alpha":
                    mx = max(sc.values())
                    t = alpha * mx if mx > 0 else mx
                    chosen = [J for J in elig if sc[J] >= t]
                else:
                    kk = math.ceil(density * len(elig) - 1e-9)
                    kk = min(len(elig), max(1, kk))
                    left = list(elig)
                    chosen = []
                    for _ in range(kk):
                        best = left[0]
                        for J in left[1:]:
                            if sc[J] > sc[best]:
                                best = J
                        chosen.append(best)
                        left.remove(best)
                    chosen.sort()
                if causal and approx and I not in chosen:
                    chosen = sorted(chosen + [I])
                mh.append(chosen)
                tail = [J for J in elig if J not in chosen] if approx else []
                for i in range(start[I], stop[I]):
                    qi = q[b][h][i]
                    terms = []   # (logit, multiplicity, value vector)
                    for J in chosen:
                        for j in range(start[J], stop[J]):
                            if causal and j > i:
                                continue
                            terms.append((scale * _dot(qi, k[b][g][j]), 1.0, v[b][g][j]))
                    for J in tail:
                        terms.append((scale * _dot(qi, kbar[J]), float(stop[J] - start[J]), vsum[J]))
                    mx = max(z for z, _, _ in terms)
                    den = 0.0
                    num = [0.0] * d
                    for z, mult, val in terms:
                        w = math.exp(z - mx)
                        den += mult * w
                        for c in range(d):
                            num[c] += w * val[c]
                    oh[i] = [x / den for x in num]
            mb.append(mh)
            ob.append(oh)
        masks.append(mb)
        outs.append(ob)
    return masks, outs
