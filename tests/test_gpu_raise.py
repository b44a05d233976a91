"""GPU parity on inputs built to move the softmax reference.

The kernels take probabilities against a per-row reference that is raised
only when a tile's scaled maximum exceeds it by more than 16 (log2 units);
the D = 64 passes without lse take row maxima only on a wave's first kept
tile and keep that reference unless a row sum or output leaves the fp32
range, which sends the workgroup through its tiles again with the raise
rule on every tile.  Random inputs rarely
raise the reference after a row's first tile, so these inputs set the score
level of every 64-key tile explicitly (one coordinate of q is 1, the same
coordinate of k carries the level; the other coordinates are small noise):

  * head 0: +20 per tile, a raise on every tile;
  * head 1: +15.5 per tile, within one of the raise threshold on every tile
    but over it only every other tile;
  * head 2: a zigzag (+45, -25, ...), raises on the rises only;
  * head 3: random tile levels in [0, 60].

Dense attention (with and without lse), sparse attention over every block,
and sparse attention over random kept lists (with and without lse, with and
without a launch plan) are compared with the fp64 oracle at the parity
bounds: outputs 2e-2 max-abs / 2e-3 mean-abs, lse 1e-3.  The largest logit
is ~111 (natural units): the fp32 dot products then carry rounding of at
most ~1e-4 after the scale, well inside the lse bound.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle

O_MAX = 2e-2
O_MEAN = 2e-3
LSE_ATOL = 1e-3
LOG2E = 1.0 / math.log(2.0)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def losa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_losa_amd as mod
    return mod


def _levels(ntiles, rng):
    """Per-head tile levels in log2 units."""
    up = 20.0 * np.arange(ntiles)
    half = 15.5 * np.arange(ntiles)
    zig = np.cumsum(np.where(np.arange(ntiles) % 2, 45.0, -25.0)) + 25.0
    rnd = rng.uniform(0.0, 60.0, ntiles)
    return [up, half, zig, rnd]


def _inputs(d, n, seed):
    rng = np.random.default_rng(seed)
    heads = 4
    ntiles = (n + 63) // 64
    c = 1.0 / math.sqrt(d)
    q = rng.normal(0.0, 0.2, (1, heads, n, d))
    k = rng.normal(0.0, 0.2, (1, heads, n, d))
    v = rng.normal(0.0, 1.0, (1, heads, n, d))
    q[..., 0] = 1.0
    for h, lev in enumerate(_levels(ntiles, rng)):
        target = lev[np.arange(n) // 64] + rng.uniform(-3.0, 0.0, n)  # log2 units
        k[0, h, :, 0] = target / (c * LOG2E)
    # the kernels and the oracle see the same bf16-representable inputs
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (q, k, v))
    return q, k, v


def _random_lists(nb, heads, rng):
    idx = np.full((1, heads, nb, nb), -1, np.int32)
    cnt = np.zeros((1, heads, nb), np.int32)
    for h in range(heads):
        for i in range(nb):
            keep = np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False))
            idx[0, h, i, :keep.size] = keep
            cnt[0, h, i] = keep.size
    return idx, cnt


def _raise_counts(q, k, d):
    """Per head: (raises after the first tile, tiles over 2^15 that do not
    raise), summed over rows -- the lazy-reference rule applied in float64
    to the scaled tile maxima (dense order), to show what the inputs drive."""
    c2 = LOG2E / math.sqrt(d)
    n = q.shape[2]
    out = []
    for h in range(q.shape[1]):
        s = (q[0, h].astype(np.float64) @ k[0, h].astype(np.float64).T) * c2
        tmax = np.stack([s[:, j:j + 64].max(axis=1) for j in range(0, n, 64)], axis=1)
        ref = tmax[:, 0].copy()
        raises = near = 0
        for t in range(1, tmax.shape[1]):
            up = tmax[:, t] > ref + 16.0
            near += int(np.sum(~up & (tmax[:, t] > ref + 15.0)))
            raises += int(np.sum(up))
            ref = np.where(up, tmax[:, t], ref)
        out.append((raises, near))
    return out


def test_inputs_drive_the_reference():
    """Not a GPU check: the inputs below raise the reference (and come
    within one of the threshold without raising) on many tiles per row."""
    for d in (64, 128):
        n = 64 * 8 + 17
        q, k, _ = _inputs(d, n, seed=700 + d)
        (r0, _), (r1, n1), (r2, _), (r3, _) = _raise_counts(q, k, d)
        assert r0 == 8 * n            # every tile after the first
        assert r1 >= 3 * n and n1 >= 3 * n
        assert r2 == 4 * n and r3 >= n  # the four rises of the zigzag


def _cmp(o, lse, o_ref, lse_ref, what):
    err = np.abs(o.astype(np.float64) - o_ref)
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, (what, float(err.max()), float(err.mean()))
    if lse is not None:
        lerr = np.abs(lse.astype(np.float64) - lse_ref).max()
        assert lerr <= LSE_ATOL, (what, float(lerr))


@pytest.mark.gpu
@pytest.mark.parametrize("blk", [64, 128])
@pytest.mark.parametrize("d", [64, 128])
def test_reference_raises_match_oracle(losa, d, blk):
    # nine 64-key tiles, the last one ragged; with 128-token blocks the last
    # block's second tile is empty
    n = 64 * 8 + 17
    nb = (n + blk - 1) // blk
    q, k, v = _inputs(d, n, seed=700 + d)
    _say(f"[raise] D{d} block {blk} N{n}: dense")
    tq, tk, tv = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))
    o, lse = losa.dense_attn(tq, tk, tv, block=blk)
    on, _ = losa.dense_attn(tq, tk, tv, block=blk, want_lse=False)
    full_idx = np.tile(np.arange(nb, dtype=np.int32), (1, 4, nb, 1))
    full_cnt = np.full((1, 4, nb), nb, np.int32)
    fi, fc = torch.from_numpy(full_idx).cuda(), torch.from_numpy(full_cnt).cuda()
    _say(f"[raise] D{d}: sparse over every block")
    so, sl = losa.sparse_attn(tq, tk, tv, fi, fc, block=blk, want_lse=True)
    sn, _ = losa.sparse_attn(tq, tk, tv, fi, fc, block=blk)
    rng = np.random.default_rng(900 + d + blk)
    idx, cnt = _random_lists(nb, 4, rng)
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    plan = losa.sparse_plan(tc, block=blk, head_dim=d)
    _say(f"[raise] D{d}: sparse over random lists")
    ro, rl = losa.sparse_attn(tq, tk, tv, ti, tc, block=blk, want_lse=True)
    rn, _ = losa.sparse_attn(tq, tk, tv, ti, tc, block=blk)
    rp, _ = losa.sparse_attn(tq, tk, tv, ti, tc, block=blk, plan=plan)
    torch.cuda.synchronize()
    # every block kept, visited in the dense order: the same arithmetic
    assert torch.equal(so, o) and torch.equal(sl, lse) and torch.equal(sn, on)
    assert torch.equal(rp, rn)
    g = {name: t.float().cpu().numpy() for name, t in
         (("o", o), ("lse", lse), ("on", on), ("ro", ro), ("rl", rl), ("rn", rn))}
    for h in range(4):
        od, ld = oracle.dense_attention(q[0, h], k[0, h], v[0, h])
        _cmp(g["o"][0, h], g["lse"][0, h], od, ld, f"D{d} b{blk} h{h} dense")
        _cmp(g["on"][0, h], None, od, None, f"D{d} b{blk} h{h} dense no-lse")
        os_, ls_ = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], idx[0, h], cnt[0, h], blk)
        _cmp(g["ro"][0, h], g["rl"][0, h], os_, ls_, f"D{d} b{blk} h{h} sparse")
        _cmp(g["rn"][0, h], None, os_, None, f"D{d} b{blk} h{h} sparse no-lse")


@pytest.mark.gpu
def test_reference_raises_fp32(losa):
    n, d, blk = 64 * 8 + 17, 64, 64
    q, k, v = _inputs(d, n, seed=777)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q, k, v))
    _say("[raise] fp32 D64: dense")
    o, lse = losa.dense_attn(tq, tk, tv, block=blk)
    torch.cuda.synchronize()
    for h in range(4):
        od, ld = oracle.dense_attention(q[0, h], k[0, h], v[0, h])
        _cmp(o[0, h].cpu().numpy(), lse[0, h].cpu().numpy(), od, ld, f"fp32 h{h} dense")


def _jump_inputs(d, n, seed):
    """Eight heads; in head o every query row scores ~0 against every key
    except two: key 64 + 8m + o (tile 1) scores +100 and key 192 + 8m' + o
    (tile 3) +110 (natural units; m, m' drawn per head), so each row's
    maximum jumps twice, far past the raise threshold, and always at key
    offset o within the eight consecutive keys a lane holds.  Taken against
    the first tile's reference those probabilities would be 2^144 and
    2^159, beyond fp32: only a raise keeps them finite."""
    rng = np.random.default_rng(seed)
    heads = 8
    c = 1.0 / math.sqrt(d)
    q = rng.normal(0.0, 0.05, (1, heads, n, d))
    k = rng.normal(0.0, 0.05, (1, heads, n, d))
    v = rng.normal(0.0, 1.0, (1, heads, n, d))
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    jumps = []
    for o in range(heads):
        j1 = 64 + 8 * int(rng.integers(0, 8)) + o
        j2 = 192 + 8 * int(rng.integers(0, 8)) + o
        k[0, o, j1, 0] = 100.0 / c
        k[0, o, j2, 0] = 110.0 / c
        jumps.append((j1, j2))
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (q, k, v))
    return q, k, v, jumps


def test_jump_inputs_place_the_maxima():
    """Not a GPU check: the row maxima of head o sit at key offset o."""
    n, d = 64 * 6 + 17, 64
    q, k, _, jumps = _jump_inputs(d, n, seed=41)
    for o, (j1, j2) in enumerate(jumps):
        s = q[0, o].astype(np.float64) @ k[0, o].astype(np.float64).T / math.sqrt(d)
        assert j1 % 8 == o and j2 % 8 == o and j1 // 64 == 1 and j2 // 64 == 3
        assert np.all(np.argmax(s, axis=1) == j2)
        assert np.all(s[:, j1] > 99.0) and np.all(s[:, j2] > 109.0)
        assert np.all(np.delete(s, [j1, j2], axis=1) < 1.0)


@pytest.mark.gpu
@pytest.mark.parametrize("blk", [64, 128])
@pytest.mark.parametrize("d", [64, 128])
def test_jump_at_every_key_offset(losa, d, blk):
    """A jump far above a row's first tile, at every key offset within a
    lane's eight keys: the D = 64 passes without lse overflow on it and
    must take their second, exact walk over the tiles (an earlier form of
    those passes tested the probabilities of keys 0 and 1 of each group of
    eight only, and the others then overflowed into the output)."""
    n = 64 * 6 + 17
    nb = (n + blk - 1) // blk
    q, k, v, _ = _jump_inputs(d, n, seed=4100 + d + blk)
    tq, tk, tv = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))
    _say(f"[jump] D{d} block {blk} N{n}: dense, sparse")
    o, lse = losa.dense_attn(tq, tk, tv, block=blk)
    on, _ = losa.dense_attn(tq, tk, tv, block=blk, want_lse=False)
    rng = np.random.default_rng(4200 + d + blk)
    idx, cnt = _random_lists(nb, 8, rng)
    # every list keeps the blocks of both jumps (and tile 0's block, so the
    # first kept tile is not the jump's)
    must = sorted({0, 64 // blk, 192 // blk})
    for h in range(8):
        for i in range(nb):
            keep = sorted(set(idx[0, h, i, :cnt[0, h, i]].tolist()) | set(must))
            idx[0, h, i, :len(keep)] = keep
            cnt[0, h, i] = len(keep)
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    rn, _ = losa.sparse_attn(tq, tk, tv, ti, tc, block=blk)
    ro, rl = losa.sparse_attn(tq, tk, tv, ti, tc, block=blk, want_lse=True)
    torch.cuda.synchronize()
    g = {name: t.float().cpu().numpy() for name, t in
         (("o", o), ("lse", lse), ("on", on), ("rn", rn), ("ro", ro), ("rl", rl))}
    for name in g:
        assert np.isfinite(g[name]).all(), (d, blk, name)
    for h in range(8):
        od, ld = oracle.dense_attention(q[0, h], k[0, h], v[0, h])
        _cmp(g["o"][0, h], g["lse"][0, h], od, ld, f"D{d} b{blk} h{h} dense")
        _cmp(g["on"][0, h], None, od, None, f"D{d} b{blk} h{h} dense no-lse")
        os_, ls_ = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], idx[0, h], cnt[0, h], blk)
        _cmp(g["rn"][0, h], None, os_, None, f"D{d} b{blk} h{h} sparse no-lse")
        _cmp(g["ro"][0, h], g["rl"][0, h], os_, ls_, f"D{d} b{blk} h{h} sparse")


@pytest.mark.gpu
@pytest.mark.parametrize("d", [64, 128])
def test_jump_in_some_heads_only(losa, d):
    """Only heads 2 and 5 carry the overflowing jumps: their workgroups take
    the second walk over the tiles, the others' do not, and every output of
    the launch matches the oracle."""
    n, blk = 64 * 6 + 17, 64
    nb = (n + blk - 1) // blk
    q, k, v, _ = _jump_inputs(d, n, seed=4300 + d)
    for h in (0, 1, 3, 4, 6, 7):  # plain heads: small scores everywhere
        k[0, h, :, 0] = 0.0
    tq, tk, tv = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))
    _say(f"[jump-some] D{d} N{n}: dense and sparse without lse")
    on, _ = losa.dense_attn(tq, tk, tv, block=blk, want_lse=False)
    rng = np.random.default_rng(4400 + d)
    idx, cnt = _random_lists(nb, 8, rng)
    for h in range(8):
        for i in range(nb):
            keep = sorted(set(idx[0, h, i, :cnt[0, h, i]].tolist()) | {0, 1, 3})
            idx[0, h, i, :len(keep)] = keep
            cnt[0, h, i] = len(keep)
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    plan = losa.sparse_plan(tc, block=blk, head_dim=d)
    rn, _ = losa.sparse_attn(tq, tk, tv, ti, tc, block=blk, plan=plan)
    torch.cuda.synchronize()
    g_on, g_rn = on.float().cpu().numpy(), rn.float().cpu().numpy()
    assert np.isfinite(g_on).all() and np.isfinite(g_rn).all()
    for h in range(8):
        od, _ = oracle.dense_attention(q[0, h], k[0, h], v[0, h])
        _cmp(g_on[0, h], None, od, None, f"D{d} h{h} dense no-lse")
        os_, _ = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], idx[0, h], cnt[0, h], blk)
        _cmp(g_rn[0, h], None, os_, None, f"D{d} h{h} sparse no-lse")
