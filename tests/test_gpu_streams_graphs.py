"""The library enqueues only kernel launches on the caller's stream (no
allocation, memset or synchronisation inside), so

  * calls on two streams at once give the same bits as the same calls one
    after the other, and
  * the construction step and a planned sparse call captured in a HIP graph
    give, on every replay with new inputs copied into the captured buffers,
    the same bits as eager calls on those inputs.

Each graph is replayed several times with eager work and synchronisations
between the replays, and every replay is checked."""

import sys

import numpy as np
import pytest
import torch

from block_sparse_attention_losa_amd import synth

pytestmark = pytest.mark.gpu

CFG = synth.small_config(n_grid=(4, 16, 20), head_dim=128, block=64, heads=3,
                         alpha=(3.0, 0.0, 1.5), seed=31)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def losa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_losa_amd as mod
    return mod


def _inputs(step):
    """Step-3 inputs of the test shape, perturbed for later steps."""
    q, k, v = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in synth.make_inputs(CFG))
    if step == 3:
        return q, k, v
    return tuple(synth.perturb_on_device(CFG, x, step, i) for i, x in enumerate((q, k, v)))


def test_two_streams_match_sequential(losa):
    blk = CFG.block
    q, k, v = _inputs(3)
    _, _, mass = losa.dense_attn_mass(q, k, v, block=blk)
    idx, cnt = losa.select(mass, 0.95)
    plan = losa.sparse_plan(cnt, block=blk, head_dim=CFG.head_dim)
    steps = [_inputs(t) for t in (4, 5)]
    _say("[streams] sequential reference")
    ref = [losa.sparse_attn(*x, idx, cnt, block=blk, want_lse=True, plan=plan) for x in steps]
    refn = [losa.sparse_attn(*x, idx, cnt, block=blk, plan=plan)[0] for x in steps]
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in ref]
    refn = [o.clone() for o in refn]
    _say("[streams] two streams at once")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, outn = [], []
    torch.cuda.synchronize()
    for s, x in zip(streams, steps):
        with torch.cuda.stream(s):
            outs.append(losa.sparse_attn(*x, idx, cnt, block=blk, want_lse=True, plan=plan))
            outn.append(losa.sparse_attn(*x, idx, cnt, block=blk, plan=plan)[0])
    torch.cuda.synchronize()
    for (o, l), (ro, rl) in zip(outs, ref):
        assert torch.equal(o, ro) and torch.equal(l, rl)
    for o, ro in zip(outn, refn):
        assert torch.equal(o, ro)


def test_graph_replays_match_eager(losa):
    blk, d = CFG.block, CFG.head_dim
    b, h, n = CFG.batch, CFG.heads, CFG.seq_len
    nb = CFG.num_blocks
    dev = torch.device("cuda")
    q0, k0, v0 = _inputs(3)
    # captured buffers (allocated before capture)
    sq, sk, sv = (torch.empty_like(x) for x in (q0, k0, v0))
    o = torch.empty_like(q0)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=dev)
    mass = torch.empty((b, h, nb, nb), dtype=torch.float32, device=dev)
    ws = torch.empty(losa.dense_attn_mass_workspace_bytes(q0, blk), dtype=torch.uint8,
                     device=dev)
    idx = torch.empty((b, h, nb, nb), dtype=torch.int32, device=dev)
    cnt = torch.empty((b, h, nb), dtype=torch.int32, device=dev)
    plan = losa.sparse_plan(torch.zeros((b, h, nb), dtype=torch.int32, device=dev), block=blk,
                            head_dim=d)
    so = torch.empty_like(q0)
    so2 = torch.empty_like(q0)
    slse = torch.empty((b, h, n), dtype=torch.float32, device=dev)

    def construction():
        losa.dense_attn_mass(sq, sk, sv, block=blk, o=o, lse=lse, mass=mass, workspace=ws)
        losa.select(mass, 0.95, idx=idx, count=cnt)
        losa.sparse_plan(cnt, block=blk, head_dim=d, plan=plan)

    def sparse():
        losa.sparse_attn(sq, sk, sv, idx, cnt, block=blk, o=so, lse=slse, plan=plan)
        losa.sparse_attn(sq, sk, sv, idx, cnt, block=blk, o=so2, plan=plan)  # no lse

    _say("[graphs] eager warm-up, then capture")
    for x, y in zip((sq, sk, sv), (q0, k0, v0)):
        x.copy_(y)
    construction()
    sparse()
    torch.cuda.synchronize()
    g_con, g_sp = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_con):
        construction()
    with torch.cuda.graph(g_sp):
        sparse()
    torch.cuda.synchronize()

    for rep, t in enumerate((3, 6, 7)):
        _say(f"[graphs] replay {rep} on step-{t} inputs")
        x = _inputs(t)
        for dst, src in zip((sq, sk, sv), x):
            dst.copy_(src)
        torch.cuda.synchronize()
        g_con.replay()
        g_sp.replay()
        torch.cuda.synchronize()
        got = [y.clone() for y in (o, lse, mass, cnt, so, slse, so2)]
        got_idx = idx.clone()
        # eager calls on the same inputs, into fresh outputs
        eo, else_, emass = losa.dense_attn_mass(*x, block=blk)
        eidx, ecnt = losa.select(emass, 0.95)
        eplan = losa.sparse_plan(ecnt, block=blk, head_dim=d)
        eso, eslse = losa.sparse_attn(*x, eidx, ecnt, block=blk, want_lse=True, plan=eplan)
        eso2, _ = losa.sparse_attn(*x, eidx, ecnt, block=blk, plan=eplan)
        torch.cuda.synchronize()
        for a, e in zip(got, (eo, else_, emass, ecnt, eso, eslse, eso2)):
            assert torch.equal(a, e), f"replay {rep}"
        c = ecnt.cpu().numpy()
        gi, ei = got_idx.cpu().numpy(), eidx.cpu().numpy()
        for bb in range(b):
            for hh in range(h):
                for i in range(nb):
                    assert np.array_equal(gi[bb, hh, i, :c[bb, hh, i]], ei[bb, hh, i, :c[bb, hh, i]])
