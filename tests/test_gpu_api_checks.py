"""The torch binding rejects caller-supplied outputs (and launch plans) of the
wrong shape or dtype before anything is launched: the C entry points take
raw device pointers and cannot see a short buffer.  Every rejected call
below raises on the host; the one accepted case runs a small dense pass
into supplied outputs and compares it with the allocating call."""

import sys

import pytest
import torch

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


@pytest.fixture(scope="module")
def qkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = torch.Generator(device="cpu").manual_seed(7)
    b, h, n, d = 1, 2, 200, 64
    return tuple(torch.randn((b, h, n, d), generator=g).to("cuda", torch.bfloat16)
                 for _ in range(3))


def test_outputs_of_wrong_shape_or_dtype_are_rejected(losa, qkv):
    q, k, v = qkv
    b, h, n, d = q.shape
    nb = losa.api.num_blocks(n, 64)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    _say("[api] dense_attn outputs")
    with pytest.raises(ValueError):
        losa.dense_attn(q, k, v, o=torch.empty((b, h, n - 1, d), dtype=q.dtype, device=dev))
    with pytest.raises(TypeError):
        losa.dense_attn(q, k, v, o=torch.empty(q.shape, **f32))
    with pytest.raises(ValueError):
        losa.dense_attn(q, k, v, lse=torch.empty((b, h, n // 2), **f32))
    with pytest.raises(TypeError):
        losa.dense_attn(q, k, v, lse=torch.empty((b, h, n), dtype=torch.float16, device=dev))
    _say("[api] block_mass / dense_attn_mass outputs")
    with pytest.raises(ValueError):
        losa.block_mass(q, k, mass=torch.empty((b, h, nb, nb - 1), **f32))
    with pytest.raises(ValueError):
        losa.block_mass(q, k, lse_scratch=torch.empty((b, h, 1), **f32))
    with pytest.raises(ValueError):
        losa.dense_attn_mass(q, k, v, mass=torch.empty((b, h, 1, nb), **f32))
    with pytest.raises(TypeError):
        losa.dense_attn_mass(q, k, v, workspace=torch.empty(1 << 20, **f32))
    _say("[api] select / select_per_row / block_mask outputs")
    mass = torch.full((b, h, nb, nb), 1.0 / nb, **f32)
    with pytest.raises(ValueError):
        losa.select(mass, 0.9, idx=torch.empty((b, h, nb, nb - 1), **i32))
    with pytest.raises(TypeError):
        losa.select(mass, 0.9, count=torch.empty((b, h, nb), dtype=torch.int64, device=dev))
    taus = torch.full((b * h * nb,), 0.9, dtype=torch.float64, device=dev)
    with pytest.raises(ValueError):
        losa.select_per_row(mass, taus, count=torch.empty((b, h), **i32))
    idx = torch.zeros((b, h, nb, nb), **i32)
    cnt = torch.ones((b, h, nb), **i32)
    with pytest.raises(TypeError):
        losa.block_mask(idx, cnt, mask=torch.empty(idx.shape, dtype=torch.bool, device=dev))
    _say("[api] retained_mass / sparse_attn outputs and plans")
    lse = torch.zeros((b, h, n), **f32)
    with pytest.raises(ValueError):
        losa.retained_mass(lse, lse, retained=torch.empty((b, h, nb + 1), **f32))
    with pytest.raises(ValueError):
        losa.sparse_attn(q, k, v, idx, cnt, o=torch.empty((b, h, n, d // 2), dtype=q.dtype,
                                                          device=dev))
    with pytest.raises(ValueError):
        losa.sparse_attn(q, k, v, idx, cnt, plan=torch.zeros(3, **i32))
    with pytest.raises(TypeError):
        losa.sparse_plan(cnt, block=64, head_dim=d, plan=torch.zeros(1 << 12, **f32))


def test_supplied_outputs_are_written(losa, qkv):
    q, k, v = qkv
    _say("[api] dense_attn into supplied outputs")
    o_ref, lse_ref = losa.dense_attn(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    o2, lse2 = losa.dense_attn(q, k, v, o=o, lse=lse)
    torch.cuda.synchronize()
    assert o2 is o and lse2 is lse
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
