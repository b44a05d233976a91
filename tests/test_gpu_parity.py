"""GPU parity of the HIP path against the fp64 oracle on small seeded inputs
that span several tiles and ragged tails.

Tolerances:
  * masses: 1e-5 absolute (fp32 accumulation);
  * attention outputs: 2e-2 max-abs and 2e-3 mean-abs (bf16 inputs and
    outputs; the output rounding alone is up to 2^-9 relative);
  * row log-sum-exp: 1e-3 absolute.  The logits are fp32 dot products of
    exactly represented inputs; with |q.k| <= 512 and D = 128 products the
    accumulated rounding is below 512 * 128 * 2^-24 ~ 4e-3 in the raw dot,
    ~3.5e-4 after the 1/sqrt(128) scale, and the lse inherits at most that;
  * selection: bit-identical counts and kept lists, the oracle deciding on
    the GPU's own fp32 masses.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_losa_amd import synth
from tests import _margins

pytestmark = pytest.mark.gpu

MASS_ATOL = 1e-5
O_MAX = 2e-2
O_MEAN = 2e-3
LSE_ATOL = 1e-3
TAUS = (0.5, 0.9, 0.95, 0.99, 0.999, 1.0)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def losa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_losa_amd as mod
    return mod


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


CASES = {
    "tiny-ref fp32": synth.CONFIGS[1],
    "N105 D64 b64 bf16": synth.small_config(n_grid=(3, 5, 7), head_dim=64, block=64),
    "N226 text D128 b64 B2H3": synth.small_config(n_grid=(4, 6, 9), text=10, heads=3, batch=2,
                                                  head_dim=128, block=64,
                                                  alpha=(4.0, 0.0, 2.0)),
    "N264 D128 b128 tail8": synth.small_config(n_grid=(3, 8, 11), head_dim=128, block=128),
    "N198 D64 b128 tail70": synth.small_config(n_grid=(2, 9, 11), head_dim=64, block=128),
    "N1 D64": synth.small_config(n_grid=(1, 1, 1), head_dim=64, block=64, alpha=(1.0, 0.0)),
    "N64 D128 exact": synth.small_config(n_grid=(2, 4, 8), head_dim=128, block=64),
    "N128 D64 b128 exact": synth.small_config(n_grid=(2, 8, 8), head_dim=64, block=128),
    "N1280 D128 b64 many tiles": synth.small_config(n_grid=(4, 16, 20), head_dim=128, block=64,
                                                    heads=3, alpha=(3.0, 0.0, 1.5)),
    "N700 fp32 D128 b128": synth.small_config(n_grid=(4, 7, 25), head_dim=128, block=128,
                                              dtype="fp32", alpha=(2.5, 0.5)),
    "N333 fp32 D64 b64": synth.small_config(n_grid=(3, 3, 37), head_dim=64, block=64,
                                            dtype="fp32", alpha=(3.0, 1.0)),
}


def _expected_plan(count, blk):
    """The launch plan the library must produce, built here from its
    description: a header naming the shape (magic, work items, nb, query
    blocks per item); the work items (one per 128 query rows of each (b, h))
    ranked by cost bucket, descending, index order within a bucket (cost =
    the larger clipped count of the item's query blocks, bucket =
    cost * 32 // (nb + 1)); runs of 16 ranks assigned in rank order to the
    XCD with the least summed cost (sum of max(cost, 1)) among those with
    room for another run (ceil(runs / 8) each; ties to the lower XCD) -- or,
    beyond 4096 runs, run c to XCD c % 8 at position c // 8; run p of XCD x
    in slots 8 * (16 p + i) + x; every other slot -1."""
    b, h, nb = count.shape
    qpw = 2 if blk == 64 else 1
    wph = (nb + qpw - 1) // qpw
    n = b * h * wph
    flat = np.clip(count.reshape(b * h, nb), 0, nb)
    cost = np.array([flat[i // wph, (i % wph) * qpw:(i % wph) * qpw + qpw].max() for i in range(n)],
                    dtype=np.int64).reshape(-1)
    bucket = np.minimum(31, cost * 32 // (nb + 1))
    ranked = sorted(range(n), key=lambda i: (-bucket[i], i))
    ch, xcds = 16, 8
    n_runs = -(-n // ch)
    cap = -(-n_runs // xcds)
    plan = np.full(4 + xcds * ch * cap, -1, np.int64)
    plan[:4] = [0x41536F4C, n, nb, qpw]
    if n_runs <= 4096:
        load, taken, run_slot = [0] * xcds, [0] * xcds, []
        for r in range(n_runs):
            rc = sum(max(int(cost[i]), 1) for i in ranked[r * ch:(r + 1) * ch])
            x = min((xx for xx in range(xcds) if taken[xx] < cap), key=lambda xx: (load[xx], xx))
            run_slot.append((taken[x], x))
            load[x] += rc
            taken[x] += 1
    else:
        run_slot = [(r // xcds, r % xcds) for r in range(n_runs)]
    for s_, item in enumerate(ranked):
        p_, x = run_slot[s_ // ch]
        plan[4 + xcds * (p_ * ch + s_ % ch) + x] = item
    return plan


def _check_plan(plan, count, blk):
    """Every slot of the library's plan equals the one built from the
    description (and so places every work item exactly once)."""
    expect = _expected_plan(count, blk)
    assert plan.shape == expect.shape
    assert np.array_equal(plan.astype(np.int64), expect)
    items = expect[4:]
    assert np.array_equal(np.sort(items[items >= 0]), np.arange(expect[1]))


def _compare_attention(o_gpu, lse_gpu, o_ref, lse_ref, what):
    """Asserts the parity bounds; returns (max-abs, mean-abs, lse error)."""
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    assert err.max() <= O_MAX, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= O_MEAN, f"{what}: mean-abs {err.mean():.3e}"
    lerr = 0.0
    if lse_gpu is not None:
        lerr = np.abs(lse_gpu.astype(np.float64) - lse_ref).max()
        assert lerr <= LSE_ATOL, f"{what}: lse err {lerr:.3e}"
    return float(err.max()), float(err.mean()), float(lerr)


class _Worst:
    """Largest error seen per quantity, for the parity-margin record."""

    def __init__(self):
        self.v = {}

    def add(self, prefix, errs):
        for key, val in zip(("o_max", "o_mean", "lse"), errs):
            self.v[prefix + key] = max(self.v.get(prefix + key, 0.0), val)

    def put(self, key, val):
        self.v[key] = max(self.v.get(key, 0.0), float(val))


@pytest.mark.parametrize("name", sorted(CASES))
def test_pipeline_matches_oracle(losa, name):
    cfg = CASES[name]
    _say(f"[parity] case {name}: N={cfg.seq_len} D={cfg.head_dim} block={cfg.block} {cfg.dtype}")
    q, k, v = synth.make_inputs(cfg)
    tq, tk, tv = (_dev(x, cfg.dtype) for x in (q, k, v))
    blk = cfg.block
    nb = cfg.num_blocks

    _say(f"[parity] {name}: dense")
    o, lse = losa.dense_attn(tq, tk, tv, block=blk)
    _say(f"[parity] {name}: block_mass")
    mass = losa.block_mass(tq, tk, block=blk, lse=lse)
    mass_own = losa.block_mass(tq, tk, block=blk)  # first pass inside
    _say(f"[parity] {name}: dense_attn_mass")
    o_f, lse_f, mass_f = losa.dense_attn_mass(tq, tk, tv, block=blk)
    # without an lse output (bf16: row sums on the matrix cores)
    o_n, _ = losa.dense_attn(tq, tk, tv, block=blk, want_lse=False)
    torch.cuda.synchronize()
    o_ng = _np(o_n)
    o_g, lse_g, mass_g = _np(o), _np(lse), _np(mass)
    assert np.array_equal(mass_g, _np(mass_own)) or np.abs(mass_g - _np(mass_own)).max() < 1e-7
    # the one-sweep construction: O and lse from the dense pass's own
    # arithmetic, masses folded from per-row block sums
    assert np.array_equal(_np(o_f), o_g) and np.array_equal(_np(lse_f), lse_g)
    mass_fg = _np(mass_f)
    assert np.abs(mass_fg - mass_g).max() <= MASS_ATOL

    worst = _Worst()
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            od, lsed = oracle.dense_attention(q[b, h], k[b, h], v[b, h])
            worst.add("dense_", _compare_attention(o_g[b, h], lse_g[b, h], od, lsed,
                                                   f"{name} dense b{b}h{h}"))
            worst.add("dense_nolse_", _compare_attention(o_ng[b, h], None, od, None,
                                                         f"{name} dense no-lse b{b}h{h}"))
            md = oracle.block_mass(q[b, h], k[b, h], blk, lse=lsed)
            merr = np.abs(mass_g[b, h].astype(np.float64) - md).max()
            assert merr <= MASS_ATOL, f"{name} mass b{b}h{h} err {merr:.3e}"
            ferr = np.abs(mass_fg[b, h].astype(np.float64) - md).max()
            assert ferr <= MASS_ATOL, f"{name} one-sweep mass b{b}h{h} err {ferr:.3e}"
            worst.put("mass", merr)
            worst.put("mass_one_sweep", ferr)

    for tau in TAUS:
        _say(f"[parity] {name}: select tau={tau}")
        idx, count = losa.select(mass, tau)
        _say(f"[parity] {name}: sparse tau={tau}")
        os_, lses = losa.sparse_attn(tq, tk, tv, idx, count, block=blk, want_lse=True)
        # the planned launch (work items longest-first) gives the same bits
        plan = losa.sparse_plan(count, block=blk)
        op_, lsep = losa.sparse_attn(tq, tk, tv, idx, count, block=blk, want_lse=True, plan=plan)
        # and without lse, planned and not (the benchmark's call)
        on_, _ = losa.sparse_attn(tq, tk, tv, idx, count, block=blk, plan=plan)
        onu, _ = losa.sparse_attn(tq, tk, tv, idx, count, block=blk)
        torch.cuda.synchronize()
        assert torch.equal(op_, os_) and torch.equal(lsep, lses), f"{name} planned tau={tau}"
        assert torch.equal(on_, onu), f"{name} planned no-lse tau={tau}"
        _check_plan(plan.cpu().numpy(), count.cpu().numpy(), blk)
        idx_g, cnt_g, os_g, lses_g = _np(idx), _np(count), _np(os_), _np(lses)
        on_g = _np(on_)
        for b in range(cfg.batch):
            for h in range(cfg.heads):
                ridx, rcnt = oracle.select(mass_g[b, h], tau)
                assert np.array_equal(cnt_g[b, h], rcnt), f"{name} counts tau={tau} b{b}h{h}"
                for i in range(nb):
                    c = rcnt[i]
                    assert np.array_equal(idx_g[b, h, i, :c], ridx[i, :c]), \
                        f"{name} idx tau={tau} b{b}h{h} row {i}"
                ref_o, ref_lse = oracle.sparse_attention(q[b, h], k[b, h], v[b, h],
                                                         idx_g[b, h], cnt_g[b, h], blk)
                worst.add("sparse_", _compare_attention(os_g[b, h], lses_g[b, h], ref_o,
                                                        ref_lse,
                                                        f"{name} sparse tau={tau} b{b}h{h}"))
                worst.add("sparse_nolse_", _compare_attention(
                    on_g[b, h], None, ref_o, None, f"{name} sparse no-lse tau={tau} b{b}h{h}"))
        if tau == 1.0:
            # every block kept, visited in the same ascending order as the
            # dense pass: the two kernels do identical arithmetic
            assert (cnt_g == nb).all()
            assert np.array_equal(os_g, o_g) and np.array_equal(lses_g, lse_g)
            assert np.array_equal(on_g, o_ng)
    _margins.record("parity", name, **worst.v)


def test_repeat_runs_are_bitwise_identical(losa):
    cfg = CASES["N1280 D128 b64 many tiles"]
    _say("[parity] determinism")
    q, k, v = (_dev(x, cfg.dtype) for x in synth.make_inputs(cfg))
    outs = []
    for _ in range(2):
        o, lse = losa.dense_attn(q, k, v, block=cfg.block)
        m = losa.block_mass(q, k, block=cfg.block, lse=lse)
        idx, cnt = losa.select(m, 0.99)
        so, slse = losa.sparse_attn(q, k, v, idx, cnt, block=cfg.block, want_lse=True)
        torch.cuda.synchronize()
        outs.append([_np(t) for t in (o, lse, m, cnt, so, slse)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


TAIL_CASES = [(d, blk, t) for d in (64, 128)
              for blk, tails in ((64, (1, 2, 17, 31, 32, 33, 63)), (128, (1, 63, 64, 65, 127)))
              for t in tails]


@pytest.mark.parametrize("d,blk,tail", TAIL_CASES)
def test_ragged_tail_sweep(losa, d, blk, tail):
    """Every path at N = 2 blocks + a tail of 1..block-1 keys (bf16): dense
    and one-sweep mass against the oracle, the selection on the GPU's masses
    bit-identical, planned sparse attention against the oracle over the
    selected lists.  N < 384, so the 256-row dense workgroups run with most
    of their rows past N."""
    n = 2 * blk + tail
    cfg = synth.small_config(n_grid=(1, 1, n), head_dim=d, block=blk, heads=2,
                             alpha=(3.0, 0.5), seed=100 + tail)
    _say(f"[parity] tail sweep N={n} D={d} block={blk}")
    q, k, v = synth.make_inputs(cfg)
    tq, tk, tv = (_dev(x, "bf16") for x in (q, k, v))
    nb = cfg.num_blocks
    o, lse, mass = losa.dense_attn_mass(tq, tk, tv, block=blk)
    idx, cnt = losa.select(mass, 0.9)
    plan = losa.sparse_plan(cnt, block=blk, head_dim=d)
    so, slse = losa.sparse_attn(tq, tk, tv, idx, cnt, block=blk, want_lse=True, plan=plan)
    sn, _ = losa.sparse_attn(tq, tk, tv, idx, cnt, block=blk, plan=plan)
    dn, _ = losa.dense_attn(tq, tk, tv, block=blk, want_lse=False)
    torch.cuda.synchronize()
    o_g, lse_g, mass_g = _np(o), _np(lse), _np(mass)
    idx_g, cnt_g, so_g, slse_g = _np(idx), _np(cnt), _np(so), _np(slse)
    sn_g, dn_g = _np(sn), _np(dn)
    for h in range(cfg.heads):
        od, lsed = oracle.dense_attention(q[0, h], k[0, h], v[0, h])
        _compare_attention(o_g[0, h], lse_g[0, h], od, lsed, f"tail N={n} dense h{h}")
        md = oracle.block_mass(q[0, h], k[0, h], blk, lse=lsed)
        merr = np.abs(mass_g[0, h].astype(np.float64) - md).max()
        assert merr <= MASS_ATOL, f"tail N={n} mass h{h} err {merr:.3e}"
        ridx, rcnt = oracle.select(mass_g[0, h], 0.9)
        assert np.array_equal(cnt_g[0, h], rcnt), f"tail N={n} counts h{h}"
        for i in range(nb):
            assert np.array_equal(idx_g[0, h, i, :rcnt[i]], ridx[i, :rcnt[i]])
        ref_o, ref_lse = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], idx_g[0, h],
                                                 cnt_g[0, h], blk)
        _compare_attention(so_g[0, h], slse_g[0, h], ref_o, ref_lse, f"tail N={n} sparse h{h}")
        _compare_attention(sn_g[0, h], None, ref_o, None, f"tail N={n} sparse no-lse h{h}")
        _compare_attention(dn_g[0, h], None, od, None, f"tail N={n} dense no-lse h{h}")


@pytest.mark.parametrize("d,blk,dtype", [(128, 64, "bf16"), (64, 128, "bf16"),
                                         (64, 64, "fp32")])
def test_sparse_arbitrary_lists(losa, d, blk, dtype):
    """Lists in any order, single blocks, the short last block alone, an
    empty list, and entries past count that must be ignored."""
    cfg = synth.small_config(n_grid=(3, 7, 13), head_dim=d, block=blk, dtype=dtype,
                             heads=2, alpha=(2.0, 0.5), seed=21)
    _say(f"[parity] arbitrary lists d={d} block={blk} {dtype}")
    q, k, v = synth.make_inputs(cfg)
    nb = cfg.num_blocks
    rng = np.random.default_rng(5)
    idx = np.zeros((1, 2, nb, nb), np.int32)
    cnt = np.zeros((1, 2, nb), np.int32)
    for h in range(2):
        for i in range(nb):
            idx[0, h, i] = rng.permutation(nb)
            cnt[0, h, i] = rng.integers(1, nb + 1)
    idx[0, 0, 0, 0], cnt[0, 0, 0] = nb - 1, 1          # the short last block alone
    idx[0, 1, 1, :2], cnt[0, 1, 1] = [nb - 1, 0], 2
    cnt[0, 1, nb - 1] = 0                               # empty list
    tq, tk, tv = (_dev(x, dtype) for x in (q, k, v))
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    o, lse = losa.sparse_attn(tq, tk, tv, ti, tc, block=blk, want_lse=True)
    on, _ = losa.sparse_attn(tq, tk, tv, ti, tc, block=blk)
    torch.cuda.synchronize()
    o_g, lse_g, on_g = _np(o), _np(lse), _np(on)
    for h in range(2):
        qbs = [i for i in range(nb) if cnt[0, h, i] > 0]
        ref_o, ref_lse = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], idx[0, h],
                                                 cnt[0, h], blk, qblocks=qbs)
        rows = np.concatenate([np.arange(i * blk, min(cfg.seq_len, (i + 1) * blk)) for i in qbs])
        _compare_attention(o_g[0, h, rows], lse_g[0, h, rows], ref_o, ref_lse, f"lists h{h}")
        _compare_attention(on_g[0, h, rows], None, ref_o, None, f"lists no-lse h{h}")
    lo = (nb - 1) * blk
    assert (o_g[0, 1, lo:] == 0).all() and np.isneginf(lse_g[0, 1, lo:]).all()
    assert (on_g[0, 1, lo:] == 0).all()


def _clean_lists(idx, cnt, nb):
    """The lists as the library reads them: the first min(max(count, 0), nb)
    entries, those outside [0, nb) dropped, each block once."""
    out_i = np.zeros_like(idx)
    out_c = np.zeros_like(cnt)
    for i in range(idx.shape[0]):
        seen = []
        for j in idx[i, :min(max(int(cnt[i]), 0), nb)]:
            if 0 <= j < nb and j not in seen:
                seen.append(int(j))
        out_i[i, :len(seen)] = seen
        out_c[i] = len(seen)
    return out_i, out_c


@pytest.mark.parametrize("d", [128, 64])
def test_sparse_partner_blocks_and_list_guarantees(losa, d):
    """Query blocks that share a workgroup (2w and 2w+1 at block 64) with
    very different lists -- one empty beside a complete one, one holding only
    the short last block -- and lists with repeated entries, entries outside
    [0, nb) and counts below 0 or above nb, which the library reads as the
    set of in-range entries among the first count (clamped) entries.  Planned
    and unplanned calls give the same bits."""
    cfg = synth.small_config(n_grid=(4, 8, 15), head_dim=d, block=64, heads=2,
                             alpha=(2.0, 0.5), seed=23)
    _say(f"[parity] partner blocks and list guarantees d={d}")
    q, k, v = synth.make_inputs(cfg)
    nb = cfg.num_blocks
    assert nb == 8 and cfg.seq_len == 480    # last block holds 32 tokens
    rng = np.random.default_rng(9)
    idx = np.zeros((1, 2, nb, nb), np.int32)
    cnt = np.zeros((1, 2, nb), np.int32)
    idx[0, 0, 0], cnt[0, 0, 0] = rng.permutation(nb), 0          # empty beside ...
    idx[0, 0, 1], cnt[0, 0, 1] = np.arange(nb)[::-1], nb         # ... a complete list
    idx[0, 0, 2, 0], cnt[0, 0, 2] = nb - 1, 1                    # the short last block only
    idx[0, 0, 3], cnt[0, 0, 3] = rng.permutation(nb), nb
    idx[0, 0, 4, :6], cnt[0, 0, 4] = [3, 3, 5, 5, 5, 3], 6       # repeats
    idx[0, 0, 5, :6], cnt[0, 0, 5] = [-1, 2, nb, 100, 4, -7], 6  # outside [0, nb)
    idx[0, 0, 6], cnt[0, 0, 6] = rng.permutation(nb), nb + 5     # count above nb
    idx[0, 0, 7], cnt[0, 0, 7] = rng.permutation(nb), -3         # count below 0
    for i in range(nb):
        idx[0, 1, i] = rng.permutation(nb)
        cnt[0, 1, i] = rng.integers(0, nb + 1)
    cnt[0, 1, 2] = 0
    cnt[0, 1, 3] = nb
    tq, tk, tv = (_dev(x, "bf16") for x in (q, k, v))
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    o, lse = losa.sparse_attn(tq, tk, tv, ti, tc, block=64, want_lse=True)
    plan = losa.sparse_plan(tc, block=64, head_dim=d)
    o2, lse2 = losa.sparse_attn(tq, tk, tv, ti, tc, block=64, want_lse=True, plan=plan)
    on, _ = losa.sparse_attn(tq, tk, tv, ti, tc, block=64)
    on2, _ = losa.sparse_attn(tq, tk, tv, ti, tc, block=64, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(on, on2)
    o_g, lse_g, on_g = _np(o), _np(lse), _np(on)
    for h in range(2):
        ci, cc = _clean_lists(idx[0, h], cnt[0, h], nb)
        qbs = [i for i in range(nb) if cc[i] > 0]
        ref_o, ref_lse = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], ci, cc, 64,
                                                 qblocks=qbs)
        rows = np.concatenate([np.arange(i * 64, min(cfg.seq_len, (i + 1) * 64)) for i in qbs])
        _compare_attention(o_g[0, h, rows], lse_g[0, h, rows], ref_o, ref_lse,
                           f"partner lists d={d} h{h}")
        _compare_attention(on_g[0, h, rows], None, ref_o, None, f"partner lists no-lse d={d} h{h}")
        for i in range(nb):
            if cc[i] == 0:
                r = slice(i * 64, min(cfg.seq_len, (i + 1) * 64))
                assert (o_g[0, h, r] == 0).all() and np.isneginf(lse_g[0, h, r]).all(), (h, i)
                assert (on_g[0, h, r] == 0).all(), (h, i)


@pytest.mark.parametrize("nkb", [1, 3, 16, 64, 65, 200, 512, 929, 1024])
def test_select_matches_oracle_on_given_masses(losa, nkb):
    _say(f"[parity] select nkb={nkb}")
    rng = np.random.default_rng(nkb)
    rows = 37
    mass = np.empty((rows, nkb), np.float32)
    tiny = np.array([1.4e-45, 4.2e-45, 1e-40, 2.5e-39], np.float32)   # float32 denormals
    for r in range(rows):
        kind = r % 5
        if kind == 0:
            x = rng.dirichlet(np.full(nkb, 0.05))
        elif kind == 1:
            x = rng.dirichlet(np.full(nkb, 5.0))
        elif kind == 2:
            x = np.full(nkb, 1.0 / nkb)          # ties everywhere
        elif kind == 3:
            x = rng.dirichlet(np.full(nkb, 0.5))
            x[rng.integers(0, nkb, max(1, nkb // 4))] = 0.0   # exact zeros
        else:
            # denormal masses, many equal, among ordinary ones (the device
            # sorts them as denormal float64 keys)
            x = rng.dirichlet(np.full(nkb, 0.5)).astype(np.float32)
            pick = rng.integers(0, nkb, max(1, nkb // 3))
            x[pick] = rng.choice(tiny, len(pick))
        mass[r] = x.astype(np.float32)
    tm = torch.from_numpy(mass).cuda()
    for tau in TAUS + (0.3, 2.0):
        idx, cnt = losa.select(tm, tau)
        torch.cuda.synchronize()
        idx_g, cnt_g = _np(idx), _np(cnt)
        ridx, rcnt = oracle.select(mass, tau)
        assert np.array_equal(cnt_g, rcnt), f"counts nkb={nkb} tau={tau}"
        for r in range(rows):
            assert np.array_equal(idx_g[r, :rcnt[r]], ridx[r, :rcnt[r]]), (nkb, tau, r)


def test_select_golden_cases(losa, golden_dir):
    import json
    import os
    cases = json.load(open(os.path.join(golden_dir, "select_worked.json")))["cases"]
    for case in cases:
        m = torch.tensor([case["masses"]], dtype=torch.float32).cuda()
        idx, cnt = losa.select(m, case["tau"])
        torch.cuda.synchronize()
        assert int(cnt[0]) == case["count"], case["name"]
        assert idx[0, :case["count"]].cpu().tolist() == case["idx"], case["name"]


def test_scale_argument(losa):
    cfg = synth.small_config(n_grid=(2, 5, 13), head_dim=64, block=64, alpha=(2.0, 1.0))
    q, k, v = synth.make_inputs(cfg)
    tq, tk, tv = (_dev(x, "bf16") for x in (q, k, v))
    o, lse = losa.dense_attn(tq, tk, tv, block=64, scale=0.05)
    torch.cuda.synchronize()
    for h in range(2):
        od, lsed = oracle.dense_attention(q[0, h], k[0, h], v[0, h], scale=0.05)
        _compare_attention(_np(o)[0, h], _np(lse)[0, h], od, lsed, f"scale h{h}")
    assert math.isfinite(float(lse.float().abs().max()))


def test_plan_of_another_shape_is_not_followed(losa):
    """A plan made for another shape with the same number of slots (8 work
    items of two heads against 12 of three, both 128 slots) passes the size
    check; its header names the other shape, so the kernel runs every work
    item in index order instead of the plan's slots: the same bits as the
    unplanned call, every row written, within the bounds of the oracle."""
    cfg = synth.small_config(n_grid=(4, 8, 15), head_dim=128, block=64, heads=3,
                             alpha=(2.0, 0.5, 3.0), seed=41)
    nb = cfg.num_blocks
    assert nb == 8
    _say("[parity] plan of another shape")
    q, k, v = synth.make_inputs(cfg)
    tq, tk, tv = (_dev(x, "bf16") for x in (q, k, v))
    mass = losa.block_mass(tq, tk, block=64)
    idx, cnt = losa.select(mass, 0.9)
    plan3 = losa.sparse_plan(cnt, block=64, head_dim=128)
    plan2 = losa.sparse_plan(cnt[:, :2].contiguous(), block=64, head_dim=128)
    assert plan2.numel() == plan3.numel()
    o_u, l_u = losa.sparse_attn(tq, tk, tv, idx, cnt, block=64, want_lse=True)
    o_p, l_p = losa.sparse_attn(tq, tk, tv, idx, cnt, block=64, want_lse=True, plan=plan3)
    o_w = torch.full_like(o_u, float("nan"))
    l_w = torch.full_like(l_u, float("nan"))
    losa.sparse_attn(tq, tk, tv, idx, cnt, block=64, o=o_w, lse=l_w, plan=plan2)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_u) and torch.equal(l_p, l_u)
    assert torch.equal(o_w, o_u) and torch.equal(l_w, l_u)
    og, lg, ig, cg = _np(o_w), _np(l_w), _np(idx), _np(cnt)
    for h in range(cfg.heads):
        ro, rl = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], ig[0, h], cg[0, h], 64)
        _compare_attention(og[0, h], lg[0, h], ro, rl, f"foreign plan h{h}")


PLAN_SHAPES = [  # (B, H, nb, block, fill): counts drawn per query block
    (1, 3, 5, 64, "random"), (2, 3, 17, 64, "random"), (1, 4, 9, 128, "random"),
    (1, 12, 512, 64, "random"), (1, 2, 40, 64, "zero"), (1, 2, 40, 64, "full"),
    (1, 256, 512, 64, "random"),   # 65536 items: 4096 runs, the most balanced
    (1, 300, 512, 64, "random"),   # 4800 runs: dealt to the XCDs in turn
]


@pytest.mark.parametrize("b,h,nb,blk,fill", PLAN_SHAPES)
def test_plan_matches_its_description(losa, b, h, nb, blk, fill):
    """The launch plan, slot by slot, against one built on the host from its
    description (cost ranking, runs assigned to the least-loaded XCD with
    room, the in-turn dealing beyond 4096 runs), on counts alone."""
    _say(f"[parity] plan B{b} H{h} nb{nb} block{blk} {fill}")
    rng = np.random.default_rng(b * 1000 + h * 10 + nb)
    if fill == "zero":
        cnt = np.zeros((b, h, nb), np.int32)
    elif fill == "full":
        cnt = np.full((b, h, nb), nb, np.int32)
    else:
        # per head a kept fraction, per query block a count around it, and a
        # few entries outside [0, nb] (clipped by the plan)
        frac = rng.uniform(0.02, 1.0, size=(b, h, 1))
        cnt = np.clip(np.round(frac * nb * rng.uniform(0.5, 1.5, size=(b, h, nb))), 0, nb)
        cnt = cnt.astype(np.int32)
        cnt.reshape(-1)[rng.integers(0, cnt.size, size=4)] = [-3, nb + 5, 0, nb]
    tc = torch.from_numpy(cnt).to("cuda")
    plan = losa.sparse_plan(tc, block=blk, head_dim=128)
    torch.cuda.synchronize()
    _check_plan(plan.cpu().numpy(), cnt, blk)
