"""The LDS-poison debug build of the library against the library itself.

``liblosa_poison.so`` (built by ``build()`` with ``LOSA_LDS_POISON``) fills
the attention kernels' LDS with all-ones words -- NaN as fp32 and bf16 -- at
the start of each walk over the tiles and every tile slot before a load
refills it.  Every read of a tile the kernels make should find the tile's
data, so each output of the path must keep its bits; a read of a slot before
its load has landed, of the wrong slot or past a tile would surface as a NaN
or a changed bit here.  The cases cover every attention pass (dense with and
without lse, the two passes of the mass map, the one-sweep construction,
sparse attention with and without lse, planned and unplanned), both head
dims and block sizes, ragged sequences, a batch of two, and inputs whose
row maxima jump far above the first tile so that the passes without lse
take their second walk over the tiles.
"""

import ctypes
import os
import sys

import numpy as np
import pytest
import torch

from block_sparse_attention_losa_amd import _lib
from block_sparse_attention_losa_amd import build as _build


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(_build.POISON_LIB):
        pytest.skip("the LDS-poison build is not there (build() makes it)")
    import block_sparse_attention_losa_amd as losa
    normal = _lib.load()
    poison = ctypes.CDLL(_build.POISON_LIB)
    for name, (res, args) in _lib.SIGNATURES.items():
        fn = getattr(poison, name)
        fn.restype = res
        fn.argtypes = args
    return losa, normal, poison


def _path(losa, q, k, v, blk, idx, cnt):
    """Every pass of the path on one input, the sparse ones over the given
    lists; returns the outputs by name."""
    out = {}
    out["dense o"], out["dense lse"] = losa.dense_attn(q, k, v, block=blk)
    out["dense o without lse"], _ = losa.dense_attn(q, k, v, block=blk, want_lse=False)
    out["mass, two passes"] = losa.block_mass(q, k, block=blk)
    o1, l1, m1 = losa.dense_attn_mass(q, k, v, block=blk)
    out["one-sweep o"], out["one-sweep lse"], out["one-sweep mass"] = o1, l1, m1
    out["select idx"], out["select count"] = losa.select(m1, 0.95)
    plan = losa.sparse_plan(cnt, block=blk, head_dim=q.shape[-1])
    out["sparse o"], out["sparse lse"] = losa.sparse_attn(q, k, v, idx, cnt, block=blk,
                                                          want_lse=True)
    out["sparse o without lse"], _ = losa.sparse_attn(q, k, v, idx, cnt, block=blk)
    out["planned sparse o without lse"], _ = losa.sparse_attn(q, k, v, idx, cnt, block=blk,
                                                              plan=plan)
    torch.cuda.synchronize()
    return out


def _inputs(case):
    from block_sparse_attention_losa_amd import synth
    d, blk, kind = case
    if kind == "jump":
        from tests.test_gpu_raise import _jump_inputs
        q, k, v, _ = _jump_inputs(d, 64 * 6 + 17, seed=4500 + d + blk)
    else:
        batch = 2 if kind == "batch" else 1
        cfg = synth.small_config(n_grid=(3, 10, 13), text=6, heads=2, batch=batch, head_dim=d,
                                 block=blk, alpha=(3.0, 0.5), seed=60 + d + blk)
        q, k, v = synth.make_inputs(cfg)
    return (torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16) for x in (q, k, v))


CASES = [(64, 64, "layer"), (128, 64, "layer"), (64, 128, "batch"), (128, 128, "layer"),
         (64, 64, "jump"), (128, 64, "jump")]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[f"D{d}-b{b}-{k}" for d, b, k in CASES])
def test_poisoned_lds_changes_no_output_bit(libs, case):
    losa, normal, poison = libs
    q, k, v = _inputs(case)
    blk = case[1]
    _say(f"[lds-poison] {case}: N{q.shape[2]} B{q.shape[0]} H{q.shape[1]}")
    _, _, mass = losa.dense_attn_mass(q, k, v, block=blk)
    idx, cnt = losa.select(mass, 0.95)
    torch.cuda.synchronize()
    ref = _path(losa, q, k, v, blk, idx, cnt)
    saved = _lib._lib
    _lib._lib = poison
    try:
        got = _path(losa, q, k, v, blk, idx, cnt)
    finally:
        _lib._lib = saved
    nbk = cnt.cpu().numpy()
    for name, a in ref.items():
        b = got[name]
        if name == "select idx":
            # entries past each row's count are unspecified
            ai, bi = a.cpu().numpy(), b.cpu().numpy()
            for r in np.ndindex(*nbk.shape):
                c = int(ref["select count"].cpu().numpy()[r])
                assert np.array_equal(ai[r][:c], bi[r][:c]), (case, name, r)
            continue
        assert torch.equal(a, b), (case, name)
        if a.is_floating_point():
            assert torch.isfinite(a.float()).all(), (case, name)


def test_poison_build_writes_lds_and_product_build_does_not():
    """Not a GPU check: compiled to gfx950 assembly, the attention kernels of
    the product build store nothing to LDS with ds_write_b128 (their tiles
    arrive by LDS-DMA loads), while the LOSA_LDS_POISON build does -- its
    poison fills -- in every kernel; so the debug build really poisons and
    the product build carries none of it."""
    import re
    import subprocess
    import tempfile
    src = os.path.join(_build.CSRC, "attn_bf16.hip")
    counts = {}
    with tempfile.TemporaryDirectory() as tmp:
        procs = {}
        for tag, extra in (("product", []), ("poison", ["-DLOSA_LDS_POISON"])):
            out = os.path.join(tmp, tag + ".s")
            cmd = [_build.hipcc()] + _build.COMMON + ["-x", "hip", f"--offload-arch={_build.ARCH}",
                   "--cuda-device-only", "-S"] + _build.DEVICE_FLAGS + extra + [src, "-o", out]
            procs[tag] = (subprocess.Popen(cmd, stdout=subprocess.DEVNULL,
                                           stderr=subprocess.DEVNULL), out)
        for tag, (proc, out) in procs.items():
            assert proc.wait(timeout=600) == 0, tag
            text = open(out).read()
            # per kernel: the count of ds_write_b128 between its label and its end
            per = {}
            for m in re.finditer(r"^(_ZN4losa16attn_bf16_kernel\w+):[^\n]*\n(.*?)^\s+\.size", text,
                                 re.S | re.M):
                per[m.group(1)] = m.group(2).count("ds_write_b128")
            counts[tag] = per
    assert counts["product"] and set(counts["product"]) == set(counts["poison"])
    assert all(c == 0 for c in counts["product"].values()), counts["product"]
    assert all(c > 0 for c in counts["poison"].values()), counts["poison"]
