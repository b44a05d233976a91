"""GPU parity of the functions over the frozen lists: per-row thresholds,
the block mask and the retained-mass (drift) diagnostic, against the oracle.

Tolerances: selection and masks bit-identical.  The retained mass is
mean_i exp(lse'_i - lse_i) of two fp32 log-sum-exps that the sparse and
dense kernels produce; with those off the oracle's by e'_i and e_i, and
every term at most 1, the kernel's result can be off by at most
max_i (|e'_i| + |e_i|) over the query block's rows, plus its own fp32
rounding (exp within 2 ulp, a sum of at most 128 terms of depth 8: below
8e-6).  The test measures e' and e on every row and asserts that bound, so
the drift diagnostic may add no error of its own beyond fp32 rounding.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_losa_amd import synth
from tests import _margins

pytestmark = pytest.mark.gpu

RETAINED_FP32 = 8e-6


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def losa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_losa_amd as mod
    return mod


def _masses(rows, nkb, seed):
    rng = np.random.default_rng(seed)
    m = np.empty((rows, nkb), np.float32)
    for r in range(rows):
        x = rng.dirichlet(np.full(nkb, (0.05, 0.5, 5.0)[r % 3]))
        if r % 5 == 4:
            x = np.full(nkb, 1.0 / nkb)
        m[r] = x.astype(np.float32)
    return m


@pytest.mark.parametrize("nkb", [1, 16, 65, 278, 512, 929])
def test_select_per_row_matches_oracle(losa, nkb):
    _say(f"[frozen] select_per_row nkb={nkb}")
    rows = 40
    mass = _masses(rows, nkb, nkb)
    rng = np.random.default_rng(7 + nkb)
    taus = rng.uniform(0.3, 0.999, rows)
    taus[:6] = [1.0, 2.0, 0.0, -1.0, np.nan, 0.99]
    tm = torch.from_numpy(mass).cuda()
    # one threshold per row
    idx, cnt = losa.select_per_row(tm, torch.from_numpy(taus).cuda(), 1)
    torch.cuda.synchronize()
    ridx, rcnt = oracle.select_rows(mass, taus)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    ig = idx.cpu().numpy()
    for r in range(rows):
        assert np.array_equal(ig[r, :rcnt[r]], ridx[r, :rcnt[r]]), (nkb, r)
    # one threshold per group of 8 rows (e.g. one per head)
    gt = taus[6:11].copy()
    idx, cnt = losa.select_per_row(tm, torch.from_numpy(gt).cuda(), 8)
    torch.cuda.synchronize()
    ridx, rcnt = oracle.select_rows(mass, np.repeat(gt, 8))
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    ig = idx.cpu().numpy()
    for r in range(rows):
        assert np.array_equal(ig[r, :rcnt[r]], ridx[r, :rcnt[r]]), (nkb, r)
    # a constant threshold array reproduces losa_select exactly
    i1, c1 = losa.select(tm, 0.95)
    i2, c2 = losa.select_per_row(tm, torch.full((rows,), 0.95, dtype=torch.float64).cuda(), 1)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    for r in range(rows):
        c = int(c1[r])
        assert torch.equal(i1[r, :c], i2[r, :c])


@pytest.mark.parametrize("nkb", [1, 7, 64, 278, 1024])
def test_block_mask_matches_oracle(losa, nkb):
    _say(f"[frozen] block_mask nkb={nkb}")
    rows = 33
    rng = np.random.default_rng(nkb)
    idx = np.stack([rng.permutation(nkb) for _ in range(rows)]).astype(np.int32)
    cnt = rng.integers(0, nkb + 1, rows).astype(np.int32)
    cnt[0] = nkb
    cnt[1] = 0
    mask = losa.block_mask(torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(mask.cpu().numpy(), oracle.block_mask(idx, cnt, nkb))


def test_block_mask_of_selected_lists(losa):
    cfg = synth.small_config(n_grid=(3, 8, 11), head_dim=64, block=64, heads=2,
                             alpha=(3.0, 0.5))
    q, k, v = synth.make_inputs(cfg)
    tq, tk = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k))
    m = losa.block_mass(tq, tk, block=64)
    idx, cnt = losa.select(m, 0.9)
    mask = losa.block_mask(idx, cnt)
    torch.cuda.synchronize()
    mk = mask.cpu().numpy()
    assert mk.shape == tuple(m.shape) and mk.dtype == np.uint8
    ref = oracle.block_mask(idx.cpu().numpy().reshape(-1, cfg.num_blocks),
                            cnt.cpu().numpy().ravel(), cfg.num_blocks)
    assert np.array_equal(mk.reshape(ref.shape), ref)
    assert (mk.sum(-1) == cnt.cpu().numpy()).all()


CASES = {
    "N226 D128 b64 text B2H3": synth.small_config(n_grid=(4, 6, 9), text=10, heads=3, batch=2,
                                                  head_dim=128, block=64,
                                                  alpha=(4.0, 0.0, 2.0)),
    "N264 D128 b128": synth.small_config(n_grid=(3, 8, 11), head_dim=128, block=128),
    "N1280 D64 b64": synth.small_config(n_grid=(4, 16, 20), head_dim=64, block=64, heads=2,
                                        alpha=(3.0, 1.0)),
}


def _retained_bound(lse_k, lse_d, ref_k, ref_d, nb, block, n):
    """Per query block: max over its rows of |e'| + |e|, plus fp32 rounding."""
    e = np.abs(lse_k.astype(np.float64) - ref_k) + np.abs(lse_d.astype(np.float64) - ref_d)
    return np.array([e[i * block:min(n, (i + 1) * block)].max() for i in range(nb)]) + \
        RETAINED_FP32


@pytest.mark.parametrize("name", sorted(CASES))
def test_retained_mass_matches_oracle(losa, name):
    cfg = CASES[name]
    _say(f"[frozen] retained mass {name}")
    q, k, v = synth.make_inputs(cfg)
    tq, tk, tv = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))
    blk, nb, n = cfg.block, cfg.num_blocks, cfg.seq_len
    _, lse = losa.dense_attn(tq, tk, tv, block=blk)
    mass = losa.block_mass(tq, tk, block=blk, lse=lse)
    idx, cnt = losa.select(mass, 0.9)
    # construction step: the lists hold at least tau of the mass
    _, lse_s = losa.sparse_attn(tq, tk, tv, idx, cnt, block=blk, want_lse=True)
    r0 = losa.retained_mass(lse_s, lse, block=blk, head_dim=cfg.head_dim)
    # a later step: perturbed inputs, frozen lists
    pq, pk, pv = (synth.perturb_on_device(cfg, x, 9, i) for i, x in enumerate((tq, tk, tv)))
    _, lse_d = losa.dense_attn(pq, pk, pv, block=blk)
    _, lse_k = losa.sparse_attn(pq, pk, pv, idx, cnt, block=blk, want_lse=True)
    r9 = losa.retained_mass(lse_k, lse_d, block=blk, head_dim=cfg.head_dim)
    torch.cuda.synchronize()
    r0g, r9g = r0.cpu().numpy(), r9.cpu().numpy()
    ig, cg = idx.cpu().numpy(), cnt.cpu().numpy()
    g = {key: t.cpu().numpy() for key, t in
         (("lse", lse), ("lse_s", lse_s), ("lse_d", lse_d), ("lse_k", lse_k))}
    ph, pkh, pvh = (x.float().cpu().numpy() for x in (pq, pk, pv))
    worst, tol_min = 0.0, 1.0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            for (qq, kk, vv, gk, gd, rg) in ((q, k, v, "lse_s", "lse", r0g),
                                             (ph, pkh, pvh, "lse_k", "lse_d", r9g)):
                ref_d = oracle.row_lse(qq[b, h], kk[b, h])
                _, ref_k = oracle.sparse_attention(qq[b, h], kk[b, h], vv[b, h], ig[b, h],
                                                   cg[b, h], blk)
                ref = oracle.retained_mass(qq[b, h], kk[b, h], ig[b, h], cg[b, h], blk,
                                           lse=ref_d)
                tol = _retained_bound(g[gk][b, h], g[gd][b, h], ref_k, ref_d, nb, blk, n)
                err = np.abs(rg[b, h] - ref)
                assert (err <= tol).all(), (name, b, h, err.max(), tol.min())
                worst, tol_min = max(worst, float(err.max())), min(tol_min, float(tol.min()))
                if rg is r0g:
                    assert (rg[b, h] >= 0.9 - tol).all(), (b, h)
    assert r9g.shape == (cfg.batch, cfg.heads, nb)
    _margins.record("frozen", name, retained=worst, retained_tol_min=tol_min)
