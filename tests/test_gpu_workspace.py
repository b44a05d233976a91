"""GPU checks of the one-sweep construction with a workspace smaller than
the full one: the call then runs several passes over runs of the heads of
one batch item, and every output (O, lse, mass) must be the same bits as
with the full workspace, and within the parity bounds of the oracle, for
contiguous, strided and packed layouts and for fp32."""

import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_losa_amd import synth

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


def _np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _sizes(losa, q, blk):
    full = losa.dense_attn_mass_workspace_bytes(q, blk)
    least = losa.dense_attn_mass_workspace_bytes(q, blk, minimum=True)
    b, h = q.shape[:2]
    # one head per pass; two heads per pass (not dividing H = 3); one batch
    # item's heads per pass; one byte short of the full size
    per_head = least
    return [least, 2 * per_head, full - 1, full], full


def _bnhd(t):
    return t.transpose(1, 2).contiguous().transpose(1, 2)


CASES = {
    "B2H3 N226 text D128 b64": (synth.small_config(n_grid=(4, 6, 9), text=10, heads=3, batch=2,
                                                   head_dim=128, block=64,
                                                   alpha=(4.0, 0.0, 2.0)), "contiguous"),
    "B2H3 N264 D64 b128 [B,N,H,D]": (synth.small_config(n_grid=(3, 8, 11), heads=3, batch=2,
                                                        head_dim=64, block=128,
                                                        alpha=(3.0, 1.0, 0.0)), "bnhd"),
    "B2H3 N333 D64 b64 fp32": (synth.small_config(n_grid=(3, 3, 37), heads=3, batch=2,
                                                  head_dim=64, block=64, dtype="fp32",
                                                  alpha=(3.0, 1.0, 2.0)), "contiguous"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_bounded_workspace_matches_full_and_oracle(losa, name):
    cfg, layout = CASES[name]
    blk = cfg.block
    _say(f"[workspace] {name}")
    qn, kn, vn = synth.make_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).cuda().to(dt) for x in (qn, kn, vn))
    if layout == "bnhd":
        q, k, v = (_bnhd(t) for t in (q, k, v))
    sizes, full = _sizes(losa, q, blk)
    outs = {}
    for size in sizes:
        ws = torch.empty(size, dtype=torch.uint8, device="cuda")
        o_buf = None
        if layout == "bnhd":
            b, h, n, d = q.shape
            o_buf = torch.empty((b, n, h, d), dtype=dt, device="cuda").transpose(1, 2)
        o, lse, mass = losa.dense_attn_mass(q, k, v, block=blk, workspace=ws, o=o_buf)
        # and without lse (the fp32 path then keeps lse in the workspace)
        o2, _, mass2 = losa.dense_attn_mass(q, k, v, block=blk, workspace=ws, want_lse=False)
        torch.cuda.synchronize()
        assert torch.equal(o2, o) and torch.equal(mass2, mass), (name, size)
        outs[size] = (o, lse, mass)
    o_f, lse_f, mass_f = outs[full]
    for size in sizes:
        o, lse, mass = outs[size]
        assert torch.equal(o, o_f) and torch.equal(lse, lse_f) and torch.equal(mass, mass_f), \
            (name, size)
    og, lg, mg = _np(o_f), _np(lse_f), _np(mass_f)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            od, lsed = oracle.dense_attention(qn[b, h], kn[b, h], vn[b, h])
            err = np.abs(og[b, h].astype(np.float64) - od)
            assert err.max() <= O_MAX and err.mean() <= O_MEAN, (name, b, h)
            assert np.abs(lg[b, h] - lsed).max() <= LSE_ATOL, (name, b, h)
            md = oracle.block_mass(qn[b, h], kn[b, h], blk, lse=lsed)
            assert np.abs(mg[b, h].astype(np.float64) - md).max() <= MASS_ATOL, (name, b, h)


def test_workspace_below_minimum_is_rejected(losa):
    cfg = synth.small_config(n_grid=(3, 8, 11), head_dim=64, block=64)
    q, k, v = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in synth.make_inputs(cfg))
    least = losa.dense_attn_mass_workspace_bytes(q, 64, minimum=True)
    ws = torch.empty(least - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(losa.LosaError):
        losa.dense_attn_mass(q, k, v, block=64, workspace=ws)
    # a budget below the minimum still gets the minimum
    o, lse, mass = losa.dense_attn_mass(q, k, v, block=64, max_workspace_bytes=1)
    o_f, lse_f, mass_f = losa.dense_attn_mass(q, k, v, block=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o_f) and torch.equal(lse, lse_f) and torch.equal(mass, mass_f)


def test_hunyuan_layer_in_two_heads_per_pass(losa):
    """The HunyuanVideo-13B layer (B1 H24 N118800 block 128), whose full
    workspace is 10.6 GB, built in passes of two heads (0.9 GB): the same
    bits as the single pass, and the registry honours a workspace cap."""
    cfg = synth.CONFIGS[4]
    _say("[workspace] HunyuanVideo layer, two heads per pass")
    q, k, v = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in synth.make_inputs(cfg))
    least = losa.dense_attn_mass_workspace_bytes(q, 128, minimum=True)
    o, lse, mass = losa.dense_attn_mass(q, k, v, block=128, max_workspace_bytes=2 * least)
    o_f, lse_f, mass_f = losa.dense_attn_mass(q, k, v, block=128)
    torch.cuda.synchronize()
    assert torch.equal(o, o_f) and torch.equal(lse, lse_f) and torch.equal(mass, mass_f)
    del o_f, lse_f, mass_f
    reg = losa.FrozenLists(block=128, threshold=0.99, max_workspace_bytes=2 * least)
    o_r = reg.construct("layer", q, k, v)
    idx, cnt = losa.select(mass, 0.99)
    torch.cuda.synchronize()
    assert torch.equal(o_r, o) and torch.equal(reg.lists("layer")[1], cnt)
