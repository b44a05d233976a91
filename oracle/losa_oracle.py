"""Plain float64 CPU oracle of the four LoSA hot-path computations.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke``
and by the ``cpu_baseline`` leg of ``bench.py``; never by the product.

Every function works on one (batch, head) slice: ``q``, ``k``, ``v`` are
``[N, D]`` arrays (any float dtype; they are upcast exactly to float64).
Nothing is blocked, fused or reordered beyond what the definitions state;
rows are processed one query block at a time only to bound memory, which does
not change any per-row result.

Notation follows the pages: ``s`` scores, ``lse`` row log-sum-exp, ``M`` the
block mass map, ``tau`` the retained-mass threshold, ``idx``/``count`` the
frozen per-(head, query block) key-block lists.

Readings taken where the pages are silent:
  * softmax scale ``c = 1/sqrt(D)`` unless given;
  * a block is ``block`` consecutive tokens of the flattened sequence; the
    last block holds the ``N - (nb-1)*block`` remaining tokens;
  * the mass of a query block is the *average* over its valid rows, so each
    row of ``M`` sums to 1 and ``tau`` is a fraction of the mass;
  * ties in the descending-mass order are broken by ascending block index;
  * "reaches the threshold" is ``S_k >= tau`` with ``S_k`` accumulated in
    float64 in sorted order; ``tau >= 1`` keeps every block, and a row whose
    total stays below ``tau`` also keeps every block;
  * sparse attention renormalises the softmax over the retained keys only.
"""

import math

import numpy as np


def num_blocks(n, block):
    """Number of (square) blocks covering ``n`` tokens: ceil(n / block)."""
    return (int(n) + int(block) - 1) // int(block)


def block_rows(index, n, block):
    """Token range ``[lo, hi)`` of block ``index`` clipped to the sequence."""
    lo = int(index) * int(block)
    return lo, min(int(n), lo + int(block))


def _scale(d, scale):
    if scale is None or scale == 0:
        return 1.0 / math.sqrt(d)
    return float(scale)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _softmax_apply(s, v):
    """Row softmax of the score block ``s`` (``-inf`` marks absent keys),
    then the weighted sum of the rows of ``v``.

    lse_i = m_i + log sum_j exp(s_ij - m_i), with m_i = max_j s_ij;
    o_i   = sum_j exp(s_ij - lse_i) v_j.
    """
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p @ v, lse


def dense_attention(q, k, v, scale=None, rows=None, chunk=64):
    """Dense softmax self-attention over all N keys (the quadratic pass the
    method runs at its early dense steps and at the construction step).

    [mlsanity.com paper index, "Abstract (arXiv)": self-attention over the
    long 3D token sequence; legiblepapers, "Summary & Methodology Analysis":
    dense self-attention for the first denoising steps.]

    Returns ``(o, lse)`` for the requested query ``rows`` (all rows by
    default): ``o`` is ``[len(rows), D]`` and ``lse`` (natural log) is
    ``[len(rows)]``, both float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    c = _scale(q.shape[1], scale)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o = np.empty((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    for a in range(0, len(rows), chunk):
        r = rows[a:a + chunk]
        s = c * (q[r] @ k.T)
        o[a:a + len(r)], lse[a:a + len(r)] = _softmax_apply(s, v)
    return o, lse


def row_lse(q, k, scale=None, rows=None, chunk=64):
    """First pass of the mass computation alone: lse_i = log sum_j exp(s_ij)."""
    q, k = _f64(q), _f64(k)
    c = _scale(q.shape[1], scale)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    lse = np.empty(len(rows))
    for a in range(0, len(rows), chunk):
        r = rows[a:a + chunk]
        s = c * (q[r] @ k.T)
        m = s.max(axis=1)
        lse[a:a + len(r)] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return lse


def block_mass(q, k, block, scale=None, lse=None, qblocks=None):
    """Exact block attention mass ("mass map") of one (batch, head).

    M[I, J] = (1/|I|) * sum_{i in I} sum_{j in J} exp(s_ij - lse_i)

    where |I| counts the valid rows of query block I and the keys of J are
    clipped to the sequence.  The row log-sum-exp is the first pass (taken
    from ``lse`` when given, as the dense pass produces it); the scores are
    then recomputed and their probabilities summed per key block.

    [mlsanity.com paper index, "Abstract (arXiv)": exact block attention
    masses measured at one early dense step; ubos.tech blog, "How It Works
    in Practice", Phase 1: the weight mass of each block pair forms a mass
    map; legiblepapers, "Summary & Methodology Analysis": per layer, head and
    query block at the construction step.]

    Returns ``[len(qblocks), nb]`` float64 (all query blocks by default).
    """
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    c = _scale(q.shape[1], scale)
    nb = num_blocks(n, block)
    if lse is None:
        lse = row_lse(q, k, scale)
    lse = _f64(lse)
    qblocks = range(nb) if qblocks is None else qblocks
    out = np.zeros((len(qblocks), nb))
    for row, qi in enumerate(qblocks):
        lo, hi = block_rows(qi, n, block)
        s = c * (q[lo:hi] @ k.T)
        p = np.exp(s - lse[lo:hi, None])
        # pad the key axis with zero probability up to nb*block, then sum
        # every (row, key) of each key block
        padded = np.zeros((hi - lo, nb * block))
        padded[:, :n] = p
        out[row] = padded.reshape(hi - lo, nb, block).sum(axis=(0, 2)) / (hi - lo)
    return out


def select_row(x, tau):
    """Threshold selection for one query block.

    Sort the key blocks by descending mass (ties: ascending block index),
    accumulate the masses in that order in float64, and keep the smallest
    prefix whose sum reaches ``tau``.  ``tau >= 1`` keeps every block, and
    so does a row whose total never reaches ``tau``.

    [ubos.tech blog, "How It Works in Practice", Phase 2: sort by descending
    mass and accumulate until the threshold is met; mlsanity.com paper index,
    "Abstract (arXiv)": the smallest key/value block set meeting the
    threshold; legiblepapers, FAQ Q4: cumulative mass threshold 0.99.]

    ``x`` holds the masses of one query block (float32 or float64; each value
    is converted exactly).  Returns ``(idx, count)`` with ``idx`` the kept
    block indices in descending-mass order.
    """
    x = [float(val) for val in np.asarray(x).ravel()]
    nb = len(x)
    order = sorted(range(nb), key=lambda j: (-x[j], j))
    count = nb
    if tau < 1.0:
        total = 0.0
        for kept, j in enumerate(order, start=1):
            total += x[j]
            if total >= tau:
                count = kept
                break
    return np.asarray(order[:count], dtype=np.int64), count


def select(mass, tau):
    """:func:`select_row` over every row of ``mass`` (``[R, nb]``).

    Returns ``idx`` ``[R, nb]`` int32 (entries at and after ``count`` are -1)
    and ``count`` ``[R]`` int32.
    """
    mass = np.asarray(mass)
    rows, nb = mass.shape
    idx = np.full((rows, nb), -1, dtype=np.int32)
    count = np.zeros(rows, dtype=np.int32)
    for r in range(rows):
        kept, cnt = select_row(mass[r], tau)
        idx[r, :cnt] = kept
        count[r] = cnt
    return idx, count


def kept_key_mask(idx_row, count, block, n):
    """Boolean ``[n]`` mask of the keys in the first ``count`` blocks of
    ``idx_row`` (token ranges clipped to the sequence)."""
    mask = np.zeros(int(n), dtype=bool)
    for j in np.asarray(idx_row)[:int(count)]:
        lo, hi = block_rows(j, n, block)
        mask[lo:hi] = True
    return mask


def sparse_attention(q, k, v, idx, count, block, scale=None, qblocks=None):
    """Block-sparse softmax attention over frozen block lists.

    For each query block I the retained keys are the tokens of the blocks
    ``idx[I, :count[I]]``; every other score is -inf, so the softmax is
    renormalised over the retained keys:

        lse'_i = log sum_{j kept} exp(s_ij),
        o_i    = sum_{j kept} exp(s_ij - lse'_i) v_j.

    [ubos.tech blog, "How It Works in Practice", Phase 3: the frozen mask
    restricts attention look-ups to the retained key/value blocks;
    legiblepapers, "Summary & Methodology Analysis": later steps attend only
    to the frozen retained keys, with Q/K/V recomputed each step.]

    ``idx`` is ``[nb, nb]`` and ``count`` ``[nb]`` for this (batch, head).
    Returns ``(o, lse)`` for the rows of ``qblocks`` (all by default), rows
    in token order.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    c = _scale(q.shape[1], scale)
    nb = num_blocks(n, block)
    qblocks = range(nb) if qblocks is None else qblocks
    o_parts, lse_parts = [], []
    for qi in qblocks:
        lo, hi = block_rows(qi, n, block)
        s = c * (q[lo:hi] @ k.T)
        s[:, ~kept_key_mask(idx[qi], count[qi], block, n)] = -np.inf
        o_blk, lse_blk = _softmax_apply(s, v)
        o_parts.append(o_blk)
        lse_parts.append(lse_blk)
    return np.concatenate(o_parts), np.concatenate(lse_parts)


def retained_mass(q, k, idx, count, block, scale=None, lse=None, qblocks=None):
    """Share of each query block's dense attention mass that falls on its
    retained keys, averaged over the block's valid rows:

        R[I] = (1/|I|) * sum_{i in I} sum_{j kept by I} exp(s_ij - lse_i)

    with ``lse`` the dense row log-sum-exp of the same inputs (computed when
    not given).  On the construction-step inputs R[I] is at least tau by
    selection; on later-step inputs it measures how much of the attention
    mass the frozen lists still cover.

    [ubos.tech blog, "Key Findings": the high-mass block set stays stable
    across denoising steps, so one early calibration serves the whole
    generation; aitobox blog, "Key Highlights": the high-mass support
    remains stable across denoising steps.]

    ``idx`` is ``[nb, nb]`` and ``count`` ``[nb]`` for this (batch, head).
    Returns ``[len(qblocks)]`` float64 (all query blocks by default).
    """
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    c = _scale(q.shape[1], scale)
    nb = num_blocks(n, block)
    if lse is None:
        lse = row_lse(q, k, scale)
    lse = _f64(lse)
    qblocks = range(nb) if qblocks is None else qblocks
    out = np.zeros(len(qblocks))
    for row, qi in enumerate(qblocks):
        lo, hi = block_rows(qi, n, block)
        s = c * (q[lo:hi] @ k.T)
        p = np.exp(s - lse[lo:hi, None])
        keep = kept_key_mask(idx[qi], count[qi], block, n)
        out[row] = p[:, keep].sum(axis=1).mean()
    return out


def select_rows(mass, taus):
    """:func:`select_row` with a threshold of its own for every row of
    ``mass`` (``[R, nb]``; ``taus`` ``[R]``).

    [ubos.tech blog, "What Comes Next": adapting the retained-mass target per
    frame or per scene.]

    Returns ``idx`` ``[R, nb]`` int32 (-1 past ``count``) and ``count``.
    """
    mass = np.asarray(mass)
    rows, nb = mass.shape
    idx = np.full((rows, nb), -1, dtype=np.int32)
    count = np.zeros(rows, dtype=np.int32)
    for r in range(rows):
        kept, cnt = select_row(mass[r], float(taus[r]))
        idx[r, :cnt] = kept
        count[r] = cnt
    return idx, count


def block_mask(idx, count, nkb):
    """The block mask: ``mask[r, j] = 1`` when key block ``j`` is among the
    first ``count[r]`` entries of ``idx[r]``, else 0 (uint8 ``[R, nkb]``).

    [ubos.tech blog, "How It Works in Practice", Phase 2: the selection
    yields a mask tensor of shape (heads, query blocks, key blocks) that is
    stored for reuse.]
    """
    idx = np.asarray(idx)
    count = np.asarray(count).ravel()
    rows = count.shape[0]
    idx = idx.reshape(rows, -1)
    mask = np.zeros((rows, int(nkb)), dtype=np.uint8)
    for r in range(rows):
        for j in idx[r, :int(count[r])]:
            mask[r, int(j)] = 1
    return mask
