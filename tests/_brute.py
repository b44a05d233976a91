"""Brute-force pure-Python versions of the hot-path definitions, for tiny
inputs only.  They use nested loops and ``math.exp``/``math.log`` on Python
floats and share nothing with the oracle's numpy code, so agreement between
the two pins the oracle's indexing, scaling and normalisation."""

import itertools
import math
from fractions import Fraction


def attention(q, k, v, scale, keep=None):
    """o_i = sum_j softmax_j(scale * <q_i, k_j>) v_j over the keys j with
    ``keep(i, j)`` true (all keys when ``keep`` is None); returns (o, lse)."""
    n, d = len(q), len(q[0])
    dv = len(v[0])
    o, lse = [], []
    for i in range(n):
        scores = []
        for j in range(len(k)):
            if keep is not None and not keep(i, j):
                continue
            dot = 0.0
            for t in range(d):
                dot += q[i][t] * k[j][t]
            scores.append((j, scale * dot))
        m = max(s for _, s in scores)
        z = 0.0
        for _, s in scores:
            z += math.exp(s - m)
        row_lse = m + math.log(z)
        out = [0.0] * dv
        for j, s in scores:
            w = math.exp(s - row_lse)
            for t in range(dv):
                out[t] += w * v[j][t]
        o.append(out)
        lse.append(row_lse)
    return o, lse


def mass(q, k, scale, block):
    """M[I][J] = average over the valid rows i of I of the attention
    probability that row i puts on the keys of J."""
    n = len(q)
    nb = (n + block - 1) // block
    _, lse = attention(q, k, [[0.0]] * len(k), scale)
    out = [[0.0] * nb for _ in range(nb)]
    for big_i in range(nb):
        rows = range(big_i * block, min(n, (big_i + 1) * block))
        for big_j in range(nb):
            total = 0.0
            for i in rows:
                for j in range(big_j * block, min(n, (big_j + 1) * block)):
                    dot = sum(q[i][t] * k[j][t] for t in range(len(q[0])))
                    total += math.exp(scale * dot - lse[i])
            out[big_i][big_j] = total / len(rows)
    return out


def minimal_sets(masses, tau):
    """Exact (rational) subset enumeration for one row of masses.

    Returns ``(size, best)``: the smallest cardinality of a set of blocks
    whose mass sum reaches ``tau``, and the set of that cardinality with the
    largest mass; among equal-mass sets the one whose sorted index tuple is
    lexicographically smallest.  ``size`` is ``len(masses)`` when no
    set reaches ``tau``.
    """
    xs = [Fraction(float(x)) for x in masses]
    tau = Fraction(float(tau))
    nb = len(xs)
    for size in range(1, nb + 1):
        best = None
        for combo in itertools.combinations(range(nb), size):
            tot = sum((xs[j] for j in combo), Fraction(0))
            if tot >= tau:
                key = (tot, tuple(-j for j in sorted(combo)))
                if best is None or key > best[0]:
                    best = (key, combo)
        if best is not None:
            return size, set(best[1])
    return nb, set(range(nb))


def retained(q, k, scale, block, idx, count):
    """R[I] = average over the valid rows i of I of the dense attention
    probability that row i puts on the keys of the blocks idx[I][:count[I]]."""
    n = len(q)
    nb = (n + block - 1) // block
    _, lse = attention(q, k, [[0.0]] * len(k), scale)
    out = []
    for big_i in range(nb):
        kept = set(int(j) for j in idx[big_i][:count[big_i]])
        rows = range(big_i * block, min(n, (big_i + 1) * block))
        total = 0.0
        for i in rows:
            for j in range(n):
                if j // block in kept:
                    dot = sum(q[i][t] * k[j][t] for t in range(len(q[0])))
                    total += math.exp(scale * dot - lse[i])
        out.append(total / len(rows))
    return out
