"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that at least one pin catches each of them."""

import os
import types

import pytest

from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "losa_oracle.py")

# (original text, mutated text, pins expected to catch it)
MUTANTS = {
    "transposed scores": (
        "s = c * (q[r] @ k.T)\n        o[a",
        "s = c * (k[r] @ q.T)\n        o[a",
        [lambda: pins.test_dense_matches_brute_force(7, 3)]),
    "missing scale": (
        "        return 1.0 / math.sqrt(d)",
        "        return 1.0",
        [lambda: pins.test_dense_matches_brute_force(7, 3),
         lambda: pins.test_dense_matches_torch_sdpa_fp64()]),
    "lse off by a constant": (
        "    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))\n    p = np.exp(s - lse[:, None])\n    return p @ v, lse",
        "    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))\n    p = np.exp(s - lse[:, None])\n    return p @ v, lse + 1e-3",
        [lambda: pins.test_dense_matches_brute_force(7, 3)]),
    "mass averaged over the full block": (
        "sum(axis=(0, 2)) / (hi - lo)",
        "sum(axis=(0, 2)) / block",
        [lambda: pins.test_mass_uniform_closed_form(200, 64),
         lambda: pins.test_mass_rows_sum_to_one(250, 64)]),
    "mass summed instead of averaged": (
        "sum(axis=(0, 2)) / (hi - lo)",
        "sum(axis=(0, 2))",
        [lambda: pins.test_mass_rows_sum_to_one(256, 64)]),
    "mass with wrong sign in exponent": (
        "p = np.exp(s - lse[lo:hi, None])",
        "p = np.exp(lse[lo:hi, None] - s)",
        [lambda: pins.test_mass_matches_brute_force(12, 4)]),
    "tie broken toward larger index": (
        "key=lambda j: (-x[j], j))",
        "key=lambda j: (-x[j], -j))",
        [lambda: pins.test_select_golden_worked_cases(
            os.path.join(os.path.dirname(SRC), "..", "tests", "golden"))]),
    "strict threshold": (
        "if total >= tau:",
        "if total > tau:",
        [lambda: pins.test_select_golden_worked_cases(
            os.path.join(os.path.dirname(SRC), "..", "tests", "golden"))]),
    "ascending sort": (
        "key=lambda j: (-x[j], j))",
        "key=lambda j: (x[j], j))",
        [lambda: pins.test_select_matches_subset_enumeration(3)]),
    "off-by-one count": (
        "count = kept\n",
        "count = kept - 1 if kept > 1 else kept\n",
        [lambda: pins.test_select_invariants_and_tau_one()]),
    "sparse mask ignores count": (
        "for j in np.asarray(idx_row)[:int(count)]:",
        "for j in np.asarray(idx_row)[:int(count) + 1]:",
        [lambda: pins.test_sparse_matches_brute_force(19, 4)]),
    "tail block not clipped": (
        "return lo, min(int(n), lo + int(block))",
        "return lo, lo + int(block)",
        [lambda: pins.test_mass_rows_sum_to_one(250, 64),
         lambda: pins.test_sparse_matches_brute_force(19, 4)]),
    "retained mass over the full block": (
        "out[row] = p[:, keep].sum(axis=1).mean()",
        "out[row] = p[:, keep].sum(axis=1).sum() / block",
        [lambda: pins.test_retained_mass_matches_brute_force(19, 4)]),
    "retained mass without the dense normaliser": (
        "p = np.exp(s - lse[lo:hi, None])\n        keep",
        "p = np.exp(s)\n        keep",
        [lambda: pins.test_retained_mass_bounds_and_construction_step()]),
    "per-row threshold of the wrong row": (
        "kept, cnt = select_row(mass[r], float(taus[r]))",
        "kept, cnt = select_row(mass[r], float(taus[r - 1]))",
        [lambda: pins.test_select_rows_matches_subset_enumeration_per_row(0)]),
    "mask past count": (
        "for j in idx[r, :int(count[r])]:",
        "for j in idx[r, :int(count[r]) + 1]:",
        [lambda: pins.test_block_mask_worked_example_and_counts()]),
}


def _load_mutant(orig, new):
    with open(SRC) as fh:
        text = fh.read()
    assert text.count(orig) >= 1, orig
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(orig, new), SRC + "(mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    orig, new, checks = MUTANTS[name]
    mutant = _load_mutant(orig, new)
    monkeypatch.setattr(pins, "oracle", mutant)
    caught = 0
    for check in checks:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught mutant {name!r}"
