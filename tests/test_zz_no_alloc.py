"""GPU check of losa_block_mass_noalloc, called through the C-ABI: its mass
map is the same bits as losa_block_mass with a caller-owned lse scratch (the
same two kernels run; only the scratch's address differs), and within 1e-5
of the oracle, on consecutive calls whose second input is smaller than the
first (the static scratch keeps the previous call's contents), and at the
largest size the scratch takes."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_losa_amd import _lib, api, synth

pytestmark = pytest.mark.gpu

MASS_ATOL = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _lib.load()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(lib, q, k, block):
    """The mass map from the no-allocation entry and from losa_block_mass
    with a caller scratch, on torch's current stream."""
    b, h, n, _ = q.shape
    nb = api.num_blocks(n, block)
    desc = api.make_desc(q, block)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    m_na = torch.full((b, h, nb, nb), float("nan"), dtype=torch.float32, device=q.device)
    m_ref = torch.empty_like(m_na)
    scratch = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    assert lib.losa_block_mass_noalloc(desc, _ptr(q), _ptr(k), _ptr(m_na), stream) == 0
    assert lib.losa_block_mass(desc, _ptr(q), _ptr(k), None, _ptr(scratch), _ptr(m_ref),
                               stream) == 0
    torch.cuda.synchronize()
    return m_na, m_ref


def test_noalloc_matches_block_mass_on_consecutive_calls(lib):
    first = synth.small_config(n_grid=(4, 16, 20), head_dim=128, block=64, heads=3,
                               alpha=(3.0, 0.0, 1.5), seed=31)
    second = synth.small_config(n_grid=(3, 8, 11), head_dim=64, block=128, heads=2,
                                alpha=(2.0, 4.0), seed=32)
    assert first.batch * first.heads * first.seq_len > second.batch * second.heads * second.seq_len
    for cfg in (first, second):
        _say(f"[noalloc] {cfg.name}")
        qn, kn, _ = synth.make_inputs(cfg)
        q, k = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (qn, kn))
        m_na, m_ref = _both(lib, q, k, cfg.block)
        assert torch.equal(m_na, m_ref), cfg.name
        mg = m_na.cpu().numpy()
        for h in range(cfg.heads):
            md = oracle.block_mass(qn[0, h], kn[0, h], cfg.block)
            err = np.abs(mg[0, h].astype(np.float64) - md).max()
            assert err <= MASS_ATOL, (cfg.name, h, err)


def test_noalloc_at_its_largest_size(lib):
    """B*H*N = LOSA_NOALLOC_MAX_ROWS exactly (64 heads of 65 536 tokens,
    1024 key blocks), then a smaller call again."""
    torch.manual_seed(5)
    h, n, d = 64, 65536, 64
    assert h * n == _lib.NOALLOC_MAX_ROWS
    _say("[noalloc] B1 H64 N65536 D64 block 64")
    q = torch.randn((1, h, n, d), device="cuda").to(torch.bfloat16)
    k = torch.randn((1, h, n, d), device="cuda").to(torch.bfloat16)
    m_na, m_ref = _both(lib, q, k, 64)
    assert torch.equal(m_na, m_ref)
    sums = m_na.double().sum(-1)
    assert float((sums - 1.0).abs().max()) < 1e-4
    del m_na, m_ref, q, k
    torch.cuda.empty_cache()
    cfg = synth.small_config(n_grid=(2, 5, 13), head_dim=64, block=64, alpha=(2.0, 1.0), seed=33)
    qn, kn, _ = synth.make_inputs(cfg)
    q, k = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (qn, kn))
    m_na, m_ref = _both(lib, q, k, 64)
    assert torch.equal(m_na, m_ref)
    mg = m_na.cpu().numpy()
    for hh in range(cfg.heads):
        md = oracle.block_mass(qn[0, hh], kn[0, hh], 64)
        assert np.abs(mg[0, hh].astype(np.float64) - md).max() <= MASS_ATOL


def test_noalloc_through_the_binding(lib):
    cfg = synth.small_config(n_grid=(3, 7, 13), head_dim=128, block=64, alpha=(3.0, 0.5), seed=34)
    qn, kn, _ = synth.make_inputs(cfg)
    q, k = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (qn, kn))
    m = api.block_mass_noalloc(q, k, block=64)
    m_ref = api.block_mass(q, k, block=64)
    torch.cuda.synchronize()
    assert torch.equal(m, m_ref)
