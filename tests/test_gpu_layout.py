"""GPU checks of the DiT integration surface.

* Attention on bfloat16 views in other layouts -- a [B, N, H, D] tensor seen
  as [B, H, N, D], and q/k/v slices of a packed [B, N, 3, H, D] projection --
  read and written in place, gives the same bits as on contiguous
  [B, H, N, D] copies (the kernels do identical arithmetic; only addresses
  change), for every entry point that takes Q/K/V.
* The per-layer registry of frozen lists reproduces the direct calls, takes
  per-head thresholds, and survives a safetensors save / load round trip.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_losa_amd import synth

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("name", sorted(CASES))
def test_strided_layouts_are_bit_identical(losa, name):
    cfg = CASES[name]
    blk = cfg.block
    _say(f"[layout] {name}")
    q, k, v = _inputs(cfg)
    o_ref, lse_ref = losa.dense_attn(q, k, v, block=blk)
    mass_ref = losa.block_mass(q, k, block=blk, lse=lse_ref)
    of_ref, lf_ref, mf_ref = losa.dense_attn_mass(q, k, v, block=blk)
    idx, cnt = losa.select(mass_ref, 0.9)
    plan = losa.sparse_plan(cnt, block=blk, head_dim=cfg.head_dim)
    os_ref, ls_ref = losa.sparse_attn(q, k, v, idx, cnt, block=blk, want_lse=True, plan=plan)
    for layout, (qs, ks, vs) in (("[B,N,H,D]", tuple(_bnhd_view(t) for t in (q, k, v))),
                                 ("packed [B,N,3,H,D]", _packed_views(q, k, v))):
        assert not qs.is_contiguous()
        for o_kind in ("contiguous", "[B,N,H,D]"):
            o_buf = None if o_kind == "contiguous" else _empty_bnhd(q)
            o, lse = losa.dense_attn(qs, ks, vs, block=blk, o=o_buf)
            assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), (layout, o_kind)
            o_buf = None if o_kind == "contiguous" else _empty_bnhd(q)
            of, lf, mf = losa.dense_attn_mass(qs, ks, vs, block=blk, o=o_buf)
            assert torch.equal(of, of_ref) and torch.equal(lf, lf_ref) and torch.equal(mf, mf_ref)
            o_buf = None if o_kind == "contiguous" else _empty_bnhd(q)
            os_, ls_ = losa.sparse_attn(qs, ks, vs, idx, cnt, block=blk, o=o_buf, want_lse=True,
                                        plan=plan)
            assert torch.equal(os_, os_ref) and torch.equal(ls_, ls_ref), (layout, o_kind)
        m = losa.block_mass(qs, ks, block=blk, lse=lse_ref)
        assert torch.equal(m, mass_ref), layout
    torch.cuda.synchronize()


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


def test_registry_matches_direct_calls(losa, tmp_path):
    cfg = synth.small_config(n_grid=(3, 10, 13), text=6, heads=2, head_dim=128, block=64,
                             alpha=(3.0, 0.0), seed=7)
    nb = cfg.num_blocks
    q, k, v = _inputs(cfg)
    lq, lk, lv = (synth.perturb_on_device(cfg, x, 4, i) for i, x in enumerate((q, k, v)))
    reg = losa.FrozenLists(block=64, threshold=0.95)
    o_c = reg.construct("blocks.0.attn", q, k, v)
    o_ref, _, mass = losa.dense_attn_mass(q, k, v, block=64)
    idx, cnt = losa.select(mass, 0.95)
    assert torch.equal(o_c, o_ref)
    ridx, rcnt = reg.lists("blocks.0.attn")
    assert torch.equal(rcnt, cnt)
    for flat in range(cnt.numel()):
        b_, h_, i_ = np.unravel_index(flat, tuple(cnt.shape))
        c = int(cnt[b_, h_, i_])
        assert torch.equal(ridx[b_, h_, i_, :c], idx[b_, h_, i_, :c])
    o1, _ = reg.attend("blocks.0.attn", lq, lk, lv)
    o1_ref, _ = losa.sparse_attn(lq, lk, lv, idx, cnt, block=64)
    assert torch.equal(o1, o1_ref)
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
    # save / load
    path = tmp_path / "frozen.safetensors"
    reg.save(path)
    back = losa.FrozenLists.load(path, device="cuda")
    o2, _ = back.attend("blocks.0.attn", lq, lk, lv)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1)
    assert torch.equal(back.lists("blocks.1.attn")[1], cnt2)
