"""Pins of the fp64 oracle against things other than itself: brute-force
loops, a library attention routine, closed forms, invariants, exact rational
subset enumeration and hand-worked golden cases."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests import _brute

RNG = np.random.default_rng(1234)


def _rand(n, d, scale=1.0):
    return RNG.standard_normal((n, d)) * scale


# ---------------------------------------------------------------- dense / lse

@pytest.mark.parametrize("n,d", [(1, 4), (7, 3), (37, 8)])
def test_dense_matches_brute_force(n, d):
    q, k, v = _rand(n, d, 2.0), _rand(n, d, 2.0), _rand(n, d)
    o, lse = oracle.dense_attention(q, k, v)
    bo, blse = _brute.attention(q.tolist(), k.tolist(), v.tolist(), 1 / math.sqrt(d))
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.row_lse(q, k), blse, rtol=0, atol=1e-12)


def test_dense_matches_torch_sdpa_fp64():
    n, d = 200, 64
    q, k, v = _rand(n, d, 1.5), _rand(n, d, 1.5), _rand(n, d)
    o, _ = oracle.dense_attention(q, k, v)
    t = [torch.from_numpy(x)[None, None] for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t)[0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_dense_closed_forms():
    n, d = 100, 16
    v = _rand(n, d)
    # Q = 0: every score is 0, so lse = log N and o = mean of V's rows
    o, lse = oracle.dense_attention(np.zeros((n, d)), _rand(n, d), v)
    np.testing.assert_allclose(lse, math.log(n), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), rtol=0, atol=1e-13)
    # V rows all equal to one vector: o_i is that vector
    row = _rand(1, d)
    o, _ = oracle.dense_attention(_rand(n, d, 3), _rand(n, d, 3), np.repeat(row, n, 0))
    np.testing.assert_allclose(o, np.repeat(row, n, 0), rtol=0, atol=1e-13)


def test_dense_probabilities_sum_to_one():
    n = 48
    q, k = _rand(n, 16, 3), _rand(n, 16, 3)
    # V = identity makes o the probability matrix itself
    p, _ = oracle.dense_attention(q, k, np.eye(n))
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
    assert (p > 0).all()


def test_explicit_scale():
    n, d = 20, 8
    q, k, v = _rand(n, d), _rand(n, d), _rand(n, d)
    o, lse = oracle.dense_attention(q, k, v, scale=0.3)
    bo, blse = _brute.attention(q.tolist(), k.tolist(), v.tolist(), 0.3)
    np.testing.assert_allclose(o, bo, atol=1e-12)
    np.testing.assert_allclose(lse, blse, atol=1e-12)


# ----------------------------------------------------------------- block mass

@pytest.mark.parametrize("n,block", [(12, 4), (13, 4), (17, 5), (5, 8)])
def test_mass_matches_brute_force(n, block):
    d = 6
    q, k = _rand(n, d, 2.0), _rand(n, d, 2.0)
    m = oracle.block_mass(q, k, block)
    bm = _brute.mass(q.tolist(), k.tolist(), 1 / math.sqrt(d), block)
    np.testing.assert_allclose(m, bm, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,block", [(256, 64), (250, 64), (1000, 128)])
def test_mass_rows_sum_to_one(n, block):
    q, k = _rand(n, 32, 2.5), _rand(n, 32, 2.5)
    m = oracle.block_mass(q, k, block)
    assert m.shape == (oracle.num_blocks(n, block),) * 2
    np.testing.assert_allclose(m.sum(1), 1.0, rtol=0, atol=1e-12)


def test_mass_uses_given_lse():
    n, block = 130, 64
    q, k, v = _rand(n, 16, 2), _rand(n, 16, 2), _rand(n, 16)
    _, lse = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(oracle.block_mass(q, k, block, lse=lse),
                               oracle.block_mass(q, k, block), rtol=0, atol=1e-14)
    sub = oracle.block_mass(q, k, block, qblocks=[2, 0])
    full = oracle.block_mass(q, k, block)
    np.testing.assert_array_equal(sub, full[[2, 0]])


@pytest.mark.parametrize("n,block", [(256, 64), (200, 64), (300, 128)])
def test_mass_uniform_closed_form(n, block):
    # Q = 0: each row spreads 1/N over every key, so M[I, J] = |J| / N
    q, k = np.zeros((n, 8)), _rand(n, 8, 4)
    m = oracle.block_mass(q, k, block)
    nb = oracle.num_blocks(n, block)
    sizes = np.array([min(n, (j + 1) * block) - j * block for j in range(nb)])
    np.testing.assert_allclose(m, np.broadcast_to(sizes / n, (nb, nb)), rtol=0, atol=1e-15)


@pytest.mark.parametrize("n,block,gamma", [(256, 64, 2.0), (230, 64, 3.0), (45, 8, 1.5)])
def test_mass_block_diagonal_closed_form(n, block, gamma):
    # q_i = k_i = gamma * e_{block(i)}: scores are c*gamma^2 inside the
    # diagonal block and 0 elsewhere, so with Z_I = |I| e^{c g^2} + N - |I|
    # M[I, I] = |I| e^{c g^2} / Z_I and M[I, J != I] = |J| / Z_I.
    nb = oracle.num_blocks(n, block)
    d = max(nb, 4)
    x = np.zeros((n, d))
    for i in range(n):
        x[i, i // block] = gamma
    c = 1 / math.sqrt(d)
    m = oracle.block_mass(x, x, block)
    sizes = np.array([min(n, (j + 1) * block) - j * block for j in range(nb)], float)
    e = math.exp(c * gamma * gamma)
    for big_i in range(nb):
        z = sizes[big_i] * e + n - sizes[big_i]
        want = sizes / z
        want[big_i] = sizes[big_i] * e / z
        np.testing.assert_allclose(m[big_i], want, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ selection

def test_select_golden_worked_cases(golden_dir):
    with open(os.path.join(golden_dir, "select_worked.json")) as fh:
        cases = json.load(fh)["cases"]
    for case in cases:
        idx, count = oracle.select_row(np.array(case["masses"], np.float32), case["tau"])
        assert count == case["count"], case["name"]
        assert idx.tolist() == case["idx"], case["name"]


@pytest.mark.parametrize("seed", range(40))
def test_select_matches_subset_enumeration(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 11))
    conc = rng.choice([0.1, 0.5, 1.0, 5.0])
    x = rng.dirichlet(np.full(nb, conc)).astype(np.float32)
    if seed % 5 == 0 and nb > 2:
        x[1] = x[0]  # force a tie
    for tau in (0.3, 0.5, 0.9, 0.95, 0.99, 0.999):
        idx, count = oracle.select_row(x, tau)
        size, best = _brute.minimal_sets(x, tau)
        if size == nb and sum(float(a) for a in x) < tau:
            assert count == nb
            continue
        assert count == size
        assert set(idx.tolist()) == best


def test_select_invariants_and_tau_one():
    rng = np.random.default_rng(7)
    for _ in range(200):
        nb = int(rng.integers(1, 64))
        x = rng.dirichlet(np.full(nb, rng.choice([0.05, 1.0, 20.0]))).astype(np.float32)
        x64 = x.astype(np.float64)
        for tau in (0.5, 0.9, 0.99):
            idx, count = oracle.select_row(x, tau)
            assert len(set(idx.tolist())) == count == len(idx)
            kept = x64[idx].sum()
            if kept >= tau:
                # dropping the last kept block falls below tau
                assert x64[idx[:-1]].sum() < tau
            else:
                assert count == nb
            # kept in non-increasing mass order
            assert (np.diff(x64[idx]) <= 0).all()
        idx, count = oracle.select_row(x, 1.0)
        assert count == nb and sorted(idx.tolist()) == list(range(nb))
        idx, count = oracle.select_row(x, 2.5)
        assert count == nb


def test_select_exact_rational_decisions():
    # float64 prefix sums of float32 masses >= 2^-30 are exact below 1, so
    # the oracle's decisions equal those made in exact rationals
    from fractions import Fraction
    rng = np.random.default_rng(3)
    for _ in range(100):
        nb = 512
        x = rng.dirichlet(np.full(nb, 0.3)).astype(np.float32)
        x = np.maximum(x, np.float32(2.0 ** -30))
        for tau in (0.9, 0.99, 0.999):
            idx, count = oracle.select_row(x, tau)
            order = sorted(range(nb), key=lambda j: (-float(x[j]), j))
            tot, want = Fraction(0), nb
            for kept, j in enumerate(order, 1):
                tot += Fraction(float(x[j]))
                if tot >= Fraction(tau):
                    want = kept
                    break
            assert count == want


def test_select_table_shapes():
    mass = np.array([[0.5, 0.25, 0.25], [0.1, 0.1, 0.8]], np.float32)
    idx, count = oracle.select(mass, 0.7)
    assert count.tolist() == [2, 1]
    assert idx[0, :2].tolist() == [0, 1] and idx[1, 0] == 2
    assert (idx[0, 2:] == -1).all() and (idx[1, 1:] == -1).all()


# ---------------------------------------------------------- sparse attention

def _random_lists(nb, rng, full=False):
    idx = np.full((nb, nb), -1, np.int64)
    count = np.zeros(nb, np.int64)
    for i in range(nb):
        c = nb if full else int(rng.integers(1, nb + 1))
        # entries after count are unspecified: fill them with real block ids
        # so that reading past count would change the result
        idx[i] = rng.permutation(nb)
        count[i] = c
    return idx, count


@pytest.mark.parametrize("n,block", [(16, 4), (19, 4), (11, 5)])
def test_sparse_matches_brute_force(n, block):
    rng = np.random.default_rng(n)
    d = 5
    q, k, v = _rand(n, d, 2.0), _rand(n, d, 2.0), _rand(n, d)
    nb = oracle.num_blocks(n, block)
    idx, count = _random_lists(nb, rng)

    def keep(i, j):
        return j // block in set(idx[i // block, :count[i // block]].tolist())

    o, lse = oracle.sparse_attention(q, k, v, idx, count, block)
    bo, blse = _brute.attention(q.tolist(), k.tolist(), v.tolist(), 1 / math.sqrt(d), keep)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def test_sparse_matches_torch_sdpa_with_block_mask():
    rng = np.random.default_rng(5)
    n, d, block = 300, 32, 64
    q, k, v = _rand(n, d, 2.0), _rand(n, d, 2.0), _rand(n, d)
    nb = oracle.num_blocks(n, block)
    idx, count = _random_lists(nb, rng)
    mask = np.zeros((n, n), bool)
    for i in range(n):
        mask[i] = oracle.kept_key_mask(idx[i // block], count[i // block], block, n)
    o, _ = oracle.sparse_attention(q, k, v, idx, count, block)
    t = [torch.from_numpy(x)[None, None] for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(
        *t, attn_mask=torch.from_numpy(mask)[None, None])[0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,block", [(256, 64), (250, 64), (300, 128)])
def test_sparse_tau_one_is_dense_bitwise(n, block):
    q, k, v = _rand(n, 16, 3), _rand(n, 16, 3), _rand(n, 16)
    m = oracle.block_mass(q, k, block)
    idx, count = oracle.select(m, 1.0)
    assert (count == m.shape[1]).all()
    o, lse = oracle.sparse_attention(q, k, v, idx, count, block)
    od, lsed = oracle.dense_attention(q, k, v, chunk=block)
    assert np.array_equal(o, od) and np.array_equal(lse, lsed)


def test_sparse_single_block_and_constant_v():
    rng = np.random.default_rng(9)
    n, d, block = 200, 8, 64
    q, k, v = _rand(n, d, 2), _rand(n, d, 2), _rand(n, d)
    nb = oracle.num_blocks(n, block)
    idx = np.full((nb, nb), -1)
    idx[:, 0] = rng.integers(0, nb, nb)
    count = np.ones(nb, int)
    o, lse = oracle.sparse_attention(q, k, v, idx, count, block)
    for i in range(nb):
        lo, hi = i * block, min(n, (i + 1) * block)
        klo, khi = idx[i, 0] * block, min(n, (idx[i, 0] + 1) * block)
        s = (q[lo:hi] @ k[klo:khi].T) / math.sqrt(d)
        p = np.exp(s) / np.exp(s).sum(1, keepdims=True)  # textbook softmax
        np.testing.assert_allclose(o[lo:hi], p @ v[klo:khi], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[lo:hi], np.log(np.exp(s).sum(1)), rtol=0, atol=1e-12)
    # V rows constant: any lists give that constant back
    row = _rand(1, d)
    idx, count = _random_lists(nb, rng)
    o, _ = oracle.sparse_attention(q, k, np.repeat(row, n, 0), idx, count, block)
    np.testing.assert_allclose(o, np.repeat(row, n, 0), rtol=0, atol=1e-13)


def test_sparse_list_order_is_irrelevant():
    rng = np.random.default_rng(11)
    n, block = 260, 64
    q, k, v = _rand(n, 16, 2), _rand(n, 16, 2), _rand(n, 16)
    nb = oracle.num_blocks(n, block)
    idx, count = _random_lists(nb, rng)
    o1, _ = oracle.sparse_attention(q, k, v, idx, count, block)
    idx2 = idx.copy()
    for i in range(nb):
        idx2[i, :count[i]] = idx[i, :count[i]][::-1]
    o2, _ = oracle.sparse_attention(q, k, v, idx2, count, block)
    assert np.array_equal(o1, o2)


# ------------------------------------------------------------ end to end

def test_threshold_retains_mass_end_to_end():
    # retained mass of the chosen lists, measured with the dense lse, is >= tau
    n, block = 512, 64
    q, k = _rand(n, 16, 3), _rand(n, 16, 3)
    m = oracle.block_mass(q, k, block)
    for tau in (0.9, 0.99):
        idx, count = oracle.select(m, tau)
        for i in range(m.shape[0]):
            assert m[i, idx[i, :count[i]]].sum() >= tau


# ------------------------------------------- retained mass (drift diagnostic)

@pytest.mark.parametrize("n,block", [(16, 4), (19, 4), (11, 5)])
def test_retained_mass_matches_brute_force(n, block):
    rng = np.random.default_rng(100 + n)
    d = 5
    q, k = _rand(n, d, 2.0), _rand(n, d, 2.0)
    nb = oracle.num_blocks(n, block)
    idx, count = _random_lists(nb, rng)
    r = oracle.retained_mass(q, k, idx, count, block)
    br = _brute.retained(q.tolist(), k.tolist(), 1 / math.sqrt(d), block, idx.tolist(),
                         count.tolist())
    np.testing.assert_allclose(r, br, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,block", [(300, 64), (256, 128)])
def test_retained_mass_is_the_kept_part_of_the_mass_map(n, block):
    # the same quantity summed per key block instead of per row
    rng = np.random.default_rng(n)
    q, k = _rand(n, 16, 3), _rand(n, 16, 3)
    nb = oracle.num_blocks(n, block)
    idx, count = _random_lists(nb, rng)
    m = oracle.block_mass(q, k, block)
    r = oracle.retained_mass(q, k, idx, count, block)
    for i in range(nb):
        assert abs(r[i] - m[i, idx[i, :count[i]]].sum()) < 1e-12


def test_retained_mass_bounds_and_construction_step():
    n, block = 450, 64
    q, k = _rand(n, 16, 3), _rand(n, 16, 3)
    nb = oracle.num_blocks(n, block)
    m = oracle.block_mass(q, k, block)
    # every block kept: all of the mass
    idx, count = oracle.select(m, 1.0)
    np.testing.assert_allclose(oracle.retained_mass(q, k, idx, count, block), 1.0,
                               rtol=0, atol=1e-12)
    # lists selected on the same inputs keep at least tau
    for tau in (0.5, 0.9, 0.99):
        idx, count = oracle.select(m, tau)
        assert (oracle.retained_mass(q, k, idx, count, block) >= tau - 1e-12).all()
    # an empty list keeps nothing
    count = np.zeros(nb, int)
    assert (oracle.retained_mass(q, k, idx, count, block) == 0).all()


# --------------------------------------------------- per-row thresholds, mask

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_rows_matches_subset_enumeration_per_row(seed):
    rng = np.random.default_rng(300 + seed)
    rows, nb = 12, 8
    mass = rng.dirichlet(np.full(nb, 0.7), size=rows)
    taus = rng.uniform(0.2, 1.1, rows)
    taus[0], taus[1] = 1.0, 0.01
    idx, count = oracle.select_rows(mass, taus)
    for r in range(rows):
        size, best = _brute.minimal_sets(mass[r], taus[r] if taus[r] < 1 else 2.0)
        assert count[r] == size, (r, taus[r])
        assert set(idx[r, :count[r]].tolist()) == best
    assert count[0] == nb and count[1] == 1 and idx[1, 0] == int(np.argmax(mass[1]))


def test_block_mask_worked_example_and_counts():
    idx = np.array([[2, 0, -1], [1, -1, -1], [0, 1, 2]])
    count = np.array([2, 1, 3])
    expect = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], np.uint8)
    assert np.array_equal(oracle.block_mask(idx, count, 3), expect)
    rng = np.random.default_rng(8)
    m = rng.dirichlet(np.full(40, 0.3), size=25)
    for tau in (0.5, 0.99, 1.0):
        idx, count = oracle.select(m, tau)
        mask = oracle.block_mask(idx, count, 40)
        assert (mask.sum(1) == count).all()
        for r in range(25):
            assert set(np.nonzero(mask[r])[0].tolist()) == set(idx[r, :count[r]].tolist())
        if tau == 1.0:
            assert (mask == 1).all()
