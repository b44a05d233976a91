"""GPU checks of the DiT integration surface.

* Attention on bfloat16 views in other layouts -- a [B, N, H, D] tensor seen
  as [B, H, N, D], and q/k/v slices of a packed [B, N, 3, H, D] projection --
  read and written in place, with O written contiguous or as [B, N, H, D]:
  every result (dense O and lse, two-pass and one-sweep masses, selection,
  planned sparse O and lse) is compared with the fp64 oracle at the parity
  bounds (outputs 2e-2 max-abs / 2e-3 mean-abs, lse 1e-3, masses 1e-5,
  selection bit-identical), and is also the same bits as on contiguous
  [B, H, N, D] copies (the kernels do identical arithmetic; only addresses
  change).
* The per-layer registry of frozen lists: its construction step, its lists
  and its sparse steps (before and after a safetensors save / load round
  trip) are compared with the oracle, and reproduce the direct calls; it
  takes per-head thresholds.
"""

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


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def losa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_losa_amd as mod
    return mod


CASES = {
    "B2H3 N226 text D128 b64": synth.small_config(n_grid=(4, 6, 9), text=10, heads=3, batch=2,
                                                  head_dim=128, block=64,
                                                  alpha=(4.0, 0.0, 2.0)),
    "B1H2 N264 D64 b128": synth.small_config(n_grid=(3, 8, 11), head_dim=64, block=128),
    "B1H2 N1280 D128 b64": synth.small_config(n_grid=(4, 16, 20), head_dim=128, block=64,
                                              alpha=(3.0, 1.0)),
}


def _inputs(cfg):
    q, k, v = synth.make_inputs(cfg)
    return tuple(torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))


def _bnhd_view(t):
    """The same values in a [B, N, H, D] buffer, seen as [B, H, N, D]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _packed_views(q, k, v):
    b, h, n, d = q.shape
    x = torch.empty((b, n, 3, h, d), dtype=q.dtype, device=q.device)
    for i, t in enumerate((q, k, v)):
        x[:, :, i] = t.transpose(1, 2)
    return tuple(x[:, :, i].transpose(1, 2) for i in range(3))


def _empty_bnhd(q):
    b, h, n, d = q.shape
    return torch.empty((b, n, h, d), dtype=q.dtype, device=q.device).transpose(1, 2)


def _np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _attn_err(o, lse, o_ref, lse_ref, what):
    """Max/mean abs error of o (and lse) against the oracle, asserted at the
    parity bounds; returns (max, mean, lse error)."""
    err = np.abs(o.astype(np.float64) - o_ref)
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, (what, err.max(), err.mean())
    lerr = 0.0
    if lse is not None:
        lerr = float(np.abs(lse.astype(np.float64) - lse_ref).max())
        assert lerr <= LSE_ATOL, (what, lerr)
    return float(err.max()), float(err.mean()), lerr


TAU = 0.9


@pytest.mark.parametrize("name", sorted(CASES))
def test_strided_layouts_match_oracle(losa, name):
    cfg = CASES[name]
    blk, nb = cfg.block, cfg.num_blocks
    _say(f"[layout] {name}")
    qn, kn, vn = synth.make_inputs(cfg)
    q, k, v = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (qn, kn, vn))
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    dense_ref = {bh: oracle.dense_attention(qn[bh], kn[bh], vn[bh]) for bh in pairs}
    mass_ref = {bh: oracle.block_mass(qn[bh], kn[bh], blk, lse=dense_ref[bh][1])
                for bh in pairs}
    # contiguous calls: every strided result must be these bits
    o_c, lse_c = losa.dense_attn(q, k, v, block=blk)
    m_c = losa.block_mass(q, k, block=blk, lse=lse_c)
    of_c, lf_c, mf_c = losa.dense_attn_mass(q, k, v, block=blk)
    idx_c, cnt_c = losa.select(mf_c, TAU)
    plan = losa.sparse_plan(cnt_c, block=blk, head_dim=cfg.head_dim)
    os_c, ls_c = losa.sparse_attn(q, k, v, idx_c, cnt_c, block=blk, want_lse=True, plan=plan)
    torch.cuda.synchronize()
    idx_g, cnt_g = idx_c.cpu().numpy(), cnt_c.cpu().numpy()
    sparse_ref = {bh: oracle.sparse_attention(qn[bh], kn[bh], vn[bh], idx_g[bh], cnt_g[bh], blk)
                  for bh in pairs}
    worst = {"o_max": 0.0, "o_mean": 0.0, "lse": 0.0, "mass": 0.0, "mass_one_sweep": 0.0,
             "sparse_o_max": 0.0, "sparse_o_mean": 0.0, "sparse_lse": 0.0}

    def note(key, val):
        worst[key] = max(worst[key], val)

    for layout, (qs, ks, vs) in (("[B,N,H,D]", tuple(_bnhd_view(t) for t in (q, k, v))),
                                 ("packed [B,N,3,H,D]", _packed_views(q, k, v))):
        assert not qs.is_contiguous()
        for o_kind in ("contiguous", "[B,N,H,D]"):
            what = f"{name} {layout} O {o_kind}"
            o_buf = None if o_kind == "contiguous" else _empty_bnhd(q)
            o, lse = losa.dense_attn(qs, ks, vs, block=blk, o=o_buf)
            o_buf = None if o_kind == "contiguous" else _empty_bnhd(q)
            of, lf, mf = losa.dense_attn_mass(qs, ks, vs, block=blk, o=o_buf)
            idx, cnt = losa.select(mf, TAU)
            o_buf = None if o_kind == "contiguous" else _empty_bnhd(q)
            os_, ls_ = losa.sparse_attn(qs, ks, vs, idx, cnt, block=blk, o=o_buf,
                                        want_lse=True, plan=plan)
            torch.cuda.synchronize()
            o_g, lse_g, of_g, lf_g, mf_g = _np(o), _np(lse), _np(of), _np(lf), _np(mf)
            ig, cg, os_g, ls_g = _np(idx), _np(cnt), _np(os_), _np(ls_)
            for bh in pairs:
                od, lsed = dense_ref[bh]
                e = _attn_err(o_g[bh], lse_g[bh], od, lsed, what + f" dense {bh}")
                note("o_max", e[0]); note("o_mean", e[1]); note("lse", e[2])
                _attn_err(of_g[bh], lf_g[bh], od, lsed, what + f" one-sweep dense {bh}")
                merr = float(np.abs(mf_g[bh].astype(np.float64) - mass_ref[bh]).max())
                assert merr <= MASS_ATOL, (what, bh, merr)
                note("mass_one_sweep", merr)
                ridx, rcnt = oracle.select(mf_g[bh], TAU)
                assert np.array_equal(cg[bh], rcnt), (what, bh)
                for i in range(nb):
                    assert np.array_equal(ig[bh][i, :rcnt[i]], ridx[i, :rcnt[i]]), (what, bh, i)
                so_ref, sl_ref = sparse_ref[bh]
                e = _attn_err(os_g[bh], ls_g[bh], so_ref, sl_ref, what + f" sparse {bh}")
                note("sparse_o_max", e[0]); note("sparse_o_mean", e[1]); note("sparse_lse", e[2])
            # and the same bits as the contiguous calls
            assert torch.equal(o, o_c) and torch.equal(lse, lse_c), what
            assert torch.equal(of, of_c) and torch.equal(lf, lf_c) and torch.equal(mf, mf_c), what
            assert torch.equal(cnt, cnt_c), what
            assert torch.equal(os_, os_c) and torch.equal(ls_, ls_c), what
        m = losa.block_mass(qs, ks, block=blk, lse=lse_c)
        torch.cuda.synchronize()
        m_g = _np(m)
        for bh in pairs:
            merr = float(np.abs(m_g[bh].astype(np.float64) - mass_ref[bh]).max())
            assert merr <= MASS_ATOL, (name, layout, bh, merr)
            note("mass", merr)
        assert torch.equal(m, m_c), layout
    _margins.record("layout", name, **worst)


def test_layout_errors(losa):
    cfg = CASES["B1H2 N264 D64 b128"]
    q, k, v = _inputs(cfg)
    with pytest.raises(ValueError):   # q, k, v in different layouts
        losa.dense_attn(_bnhd_view(q), k, v, block=128)
    with pytest.raises(ValueError):   # head dim not contiguous
        losa.dense_attn(q.transpose(2, 3).contiguous().transpose(2, 3), k, v, block=128)
    qf = q.float()
    with pytest.raises(TypeError):    # fp32 views must be contiguous
        losa.dense_attn(_bnhd_view(qf), _bnhd_view(k.float()), _bnhd_view(v.float()), block=128)


def test_registry_matches_oracle_and_direct_calls(losa, tmp_path):
    cfg = synth.small_config(n_grid=(3, 10, 13), text=6, heads=2, head_dim=128, block=64,
                             alpha=(3.0, 0.0), seed=7)
    nb = cfg.num_blocks
    _say("[layout] registry")
    qn, kn, vn = synth.make_inputs(cfg)
    q, k, v = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (qn, kn, vn))
    lq, lk, lv = (synth.perturb_on_device(cfg, x, 4, i) for i, x in enumerate((q, k, v)))
    lqn, lkn, lvn = (_np(x) for x in (lq, lk, lv))
    reg = losa.FrozenLists(block=64, threshold=0.95)
    o_c = reg.construct("blocks.0.attn", q, k, v)
    o_ref, _, mass = losa.dense_attn_mass(q, k, v, block=64)
    idx, cnt = losa.select(mass, 0.95)
    o1, l1 = reg.attend("blocks.0.attn", lq, lk, lv, want_lse=True)
    o1_ref, _ = losa.sparse_attn(lq, lk, lv, idx, cnt, block=64, want_lse=True)
    o1n, _ = reg.attend("blocks.0.attn", lq, lk, lv)
    o1n_ref, _ = losa.sparse_attn(lq, lk, lv, idx, cnt, block=64)
    torch.cuda.synchronize()
    ridx, rcnt = reg.lists("blocks.0.attn")
    ri_g, rc_g, m_g = _np(ridx), _np(rcnt), _np(mass)
    o_g, o1_g, l1_g, o1n_g = _np(o_c), _np(o1), _np(l1), _np(o1n)
    for h in range(cfg.heads):
        # construction step: the dense output and the lists against the oracle
        od, lsed = oracle.dense_attention(qn[0, h], kn[0, h], vn[0, h])
        _attn_err(o_g[0, h], None, od, lsed, f"registry construct h{h}")
        md = oracle.block_mass(qn[0, h], kn[0, h], 64, lse=lsed)
        assert np.abs(m_g[0, h].astype(np.float64) - md).max() <= MASS_ATOL
        sidx, scnt = oracle.select(m_g[0, h], 0.95)
        assert np.array_equal(rc_g[0, h], scnt), h
        for i in range(nb):
            assert np.array_equal(ri_g[0, h, i, :scnt[i]], sidx[i, :scnt[i]]), (h, i)
        # a later step over the frozen lists
        so, sl = oracle.sparse_attention(lqn[0, h], lkn[0, h], lvn[0, h], ri_g[0, h],
                                         rc_g[0, h], 64)
        _attn_err(o1_g[0, h], l1_g[0, h], so, sl, f"registry attend h{h}")
        _attn_err(o1n_g[0, h], None, so, sl, f"registry attend no-lse h{h}")
    # the registry reproduces the direct calls
    assert torch.equal(o_c, o_ref)
    assert torch.equal(rcnt, cnt)
    for flat in range(cnt.numel()):
        b_, h_, i_ = np.unravel_index(flat, tuple(cnt.shape))
        c = int(cnt[b_, h_, i_])
        assert torch.equal(ridx[b_, h_, i_, :c], idx[b_, h_, i_, :c])
    assert torch.equal(o1, o1_ref) and torch.equal(o1n, o1n_ref)
    assert torch.equal(reg.mask("blocks.0.attn"), losa.block_mask(idx, cnt))
    ret = reg.retained_mass("blocks.0.attn", lq, lk, lv)
    assert ret.shape == (1, 2, nb) and float(ret.min()) >= 0.0
    # per-head thresholds
    taus = torch.tensor([0.9, 0.999], dtype=torch.float64, device=q.device)
    reg.construct("blocks.1.attn", q, k, v, threshold=taus, rows_per_threshold=nb)
    idx2, cnt2 = losa.select_per_row(mass, taus, nb)
    assert torch.equal(reg.lists("blocks.1.attn")[1], cnt2)
    c2 = cnt2.cpu().numpy()
    r = oracle.select_rows(mass.cpu().numpy().reshape(-1, nb), np.repeat(taus.cpu().numpy(), nb))
    assert np.array_equal(c2.ravel(), r[1])
    o3, l3 = reg.attend("blocks.1.attn", lq, lk, lv, want_lse=True)
    # save / load: the reloaded lists serve the same sparse steps
    path = tmp_path / "frozen.safetensors"
    reg.save(path)
    back = losa.FrozenLists.load(path, device="cuda")
    o2, l2 = back.attend("blocks.0.attn", lq, lk, lv, want_lse=True)
    o4, l4 = back.attend("blocks.1.attn", lq, lk, lv, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1) and torch.equal(l2, l1)
    assert torch.equal(o4, o3) and torch.equal(l4, l3)
    assert torch.equal(back.lists("blocks.1.attn")[1], cnt2)
    bi, bc = (_np(t) for t in back.lists("blocks.1.attn"))
    o2_g, l2_g, o4_g, l4_g = _np(o2), _np(l2), _np(o4), _np(l4)
    worst = [0.0, 0.0, 0.0]
    for h in range(cfg.heads):
        so, sl = oracle.sparse_attention(lqn[0, h], lkn[0, h], lvn[0, h], ri_g[0, h],
                                         rc_g[0, h], 64)
        e = _attn_err(o2_g[0, h], l2_g[0, h], so, sl, f"reloaded attend h{h}")
        worst = [max(a, b) for a, b in zip(worst, e)]
        so, sl = oracle.sparse_attention(lqn[0, h], lkn[0, h], lvn[0, h], bi[0, h], bc[0, h], 64)
        e = _attn_err(o4_g[0, h], l4_g[0, h], so, sl, f"reloaded per-head attend h{h}")
        worst = [max(a, b) for a, b in zip(worst, e)]
    _margins.record("layout", "registry reloaded", o_max=worst[0], o_mean=worst[1],
                    lse=worst[2])
