"""Seeded random shapes through every path, each result against the oracle.

Each case draws a batch and head count, a sequence length (ragged or not),
a head dim, a block size, the element type, a memory layout (contiguous,
[B, N, H, D] or q/k/v slices of a packed projection for bf16), per-head
positional strengths, a threshold and a workspace size, then runs: dense
attention with and without lse, the two-pass and one-sweep mass maps (the
latter in the drawn workspace), selection, the launch plan, and planned
sparse attention with and without lse -- and compares every output with
the fp64 oracle at the parity bounds (outputs 2e-2 max-abs / 2e-3 mean-abs,
lse 1e-3, masses 1e-5, selection bit-identical).
"""

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


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128]))
    blk = int(rng.choice([64, 128]))
    batch, heads = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    dtype = "fp32" if rng.random() < 0.2 else "bf16"
    grid = (int(rng.integers(1, 4)), int(rng.integers(1, 17)), int(rng.integers(1, 31)))
    text = int(rng.integers(0, 40)) if rng.random() < 0.3 else 0
    alpha = tuple(float(a) for a in rng.uniform(0.0, 4.0, heads))
    cfg = synth.small_config(n_grid=grid, text=text, heads=heads, batch=batch, head_dim=d,
                             block=blk, dtype=dtype, alpha=alpha, seed=2000 + seed)
    layout = "contiguous" if dtype == "fp32" else str(rng.choice(["contiguous", "bnhd",
                                                                   "packed"]))
    tau = float(rng.choice([0.5, 0.9, 0.95, 0.99, 0.999, 1.0]))
    ws_frac = float(rng.choice([0.0, 0.5, 1.0]))   # workspace: minimum, between, full
    return cfg, layout, tau, ws_frac


def _views(q, k, v, layout):
    if layout == "bnhd":
        return tuple(t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    if layout == "packed":
        b, h, n, d = q.shape
        x = torch.empty((b, n, 3, h, d), dtype=q.dtype, device=q.device)
        for i, t in enumerate((q, k, v)):
            x[:, :, i] = t.transpose(1, 2)
        return tuple(x[:, :, i].transpose(1, 2) for i in range(3))
    return q, k, v


def _cmp(o, lse, o_ref, lse_ref, what):
    err = np.abs(o.astype(np.float64) - o_ref)
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, (what, err.max(), err.mean())
    if lse is not None:
        assert np.abs(lse.astype(np.float64) - lse_ref).max() <= LSE_ATOL, what


@pytest.mark.parametrize("seed", range(48))
def test_random_case_matches_oracle(losa, seed):
    cfg, layout, tau, ws_frac = _case(seed)
    blk, nb, n = cfg.block, cfg.num_blocks, cfg.seq_len
    _say(f"[fuzz] seed {seed}: B{cfg.batch} H{cfg.heads} N{n} D{cfg.head_dim} block {blk} "
         f"{cfg.dtype} {layout} tau {tau} workspace {ws_frac}")
    qn, kn, vn = synth.make_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = _views(*(torch.from_numpy(x).cuda().to(dt) for x in (qn, kn, vn)), layout)
    full = losa.dense_attn_mass_workspace_bytes(q, blk)
    least = losa.dense_attn_mass_workspace_bytes(q, blk, minimum=True)
    ws = torch.empty(int(least + ws_frac * (full - least)), dtype=torch.uint8, device="cuda")

    o, lse = losa.dense_attn(q, k, v, block=blk)
    on, _ = losa.dense_attn(q, k, v, block=blk, want_lse=False)
    mass2 = losa.block_mass(q, k, block=blk)
    of, lf, mass = losa.dense_attn_mass(q, k, v, block=blk, workspace=ws)
    idx, cnt = losa.select(mass, tau)
    plan = losa.sparse_plan(cnt, block=blk, head_dim=cfg.head_dim)
    so, sl = losa.sparse_attn(q, k, v, idx, cnt, block=blk, want_lse=True, plan=plan)
    sn, _ = losa.sparse_attn(q, k, v, idx, cnt, block=blk, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(of, o) and torch.equal(lf, lse)
    g = {key: _np(t) for key, t in (("o", o), ("lse", lse), ("on", on), ("m2", mass2),
                                    ("m", mass), ("idx", idx), ("cnt", cnt), ("so", so),
                                    ("sl", sl), ("sn", sn))}
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            what = f"seed {seed} b{b} h{h}"
            od, lsed = oracle.dense_attention(qn[b, h], kn[b, h], vn[b, h])
            _cmp(g["o"][b, h], g["lse"][b, h], od, lsed, what + " dense")
            _cmp(g["on"][b, h], None, od, None, what + " dense no-lse")
            md = oracle.block_mass(qn[b, h], kn[b, h], blk, lse=lsed)
            assert np.abs(g["m"][b, h].astype(np.float64) - md).max() <= MASS_ATOL, what
            assert np.abs(g["m2"][b, h].astype(np.float64) - md).max() <= MASS_ATOL, what
            ridx, rcnt = oracle.select(g["m"][b, h], tau)
            assert np.array_equal(g["cnt"][b, h], rcnt), what
            for i in range(nb):
                assert np.array_equal(g["idx"][b, h, i, :rcnt[i]], ridx[i, :rcnt[i]]), (what, i)
            ro, rl = oracle.sparse_attention(qn[b, h], kn[b, h], vn[b, h], g["idx"][b, h],
                                             g["cnt"][b, h], blk)
            _cmp(g["so"][b, h], g["sl"][b, h], ro, rl, what + " sparse")
            _cmp(g["sn"][b, h], None, ro, None, what + " sparse no-lse")
