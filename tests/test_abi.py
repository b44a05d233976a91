"""CPU-side checks of the C-ABI library: it loads, exports every entry point
that include/losa.h declares, and rejects bad arguments before launching
anything (no GPU needed: every call below fails validation on the host)."""

import ctypes
import os
import re

import pytest

from block_sparse_attention_losa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "losa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="liblosa.so not built")

FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p(0x10002)        # misaligned
NULL = None


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(losa_[a-z_]+)\s*\(", text)))


def desc(**kw):
    base = dict(batch=1, heads=2, seq_len=1000, head_dim=128, block=64, dtype=0, scale=0.0)
    base.update(kw)
    return _lib.AttnDesc(**base)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"losa_dense_attn", "losa_block_mass", "losa_select", "losa_sparse_attn"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of date"


def test_status_strings_and_version(lib):
    for code in range(10):
        assert lib.losa_status_string(code) != b"unknown status"
    assert lib.losa_status_string(99) == b"unknown status"
    assert lib.losa_version() >= 100


def test_num_blocks(lib):
    assert lib.losa_num_blocks(desc(seq_len=32760, block=64)) == 512
    assert lib.losa_num_blocks(desc(seq_len=118800, block=128)) == 929
    assert lib.losa_num_blocks(desc(seq_len=64, block=64)) == 1
    assert lib.losa_num_blocks(None) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), 2), (dict(block=32), 2), (dict(seq_len=0), 2), (dict(batch=0), 2),
    (dict(heads=-1), 2), (dict(seq_len=1024 * 64 + 1), 2), (dict(dtype=5), 3),
    (dict(scale=-1.0), 7), (dict(scale=float("nan")), 7), (dict(scale=float("inf")), 7),
])
def test_descriptor_validation(lib, kw, code):
    d = desc(**kw)
    assert lib.losa_dense_attn(d, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == code
    assert lib.losa_sparse_attn(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == code
    assert lib.losa_block_mass(d, FAKE, FAKE, FAKE, NULL, FAKE, NULL) == code
    assert lib.losa_dense_attn_mass(d, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 1 << 40,
                                    NULL) == code
    assert lib.losa_dense_attn_mass_workspace(d) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(stride_token=64), 7),                                  # token stride < D
    (dict(stride_batch=8, stride_head=8), 7),                    # token stride missing
    (dict(stride_batch=16 * 128 * 1000, stride_head=128, stride_token=2 * 128 + 4), 5),
    (dict(stride_batch=16 * 128 * 1000, stride_head=132, stride_token=2 * 128), 5),
    (dict(dtype=1, stride_batch=2 * 128 * 1000, stride_head=128, stride_token=2 * 128), 7),
    (dict(o_stride_token=100), 7),
    (dict(batch=2, o_stride_batch=-8, o_stride_head=128, o_stride_token=256), 7),
    (dict(seq_len=60000, stride_batch=8, stride_head=8, stride_token=8 * 4096), 2),
    # output layouts in which two elements would share an address
    (dict(o_stride_token=128), 7),                               # heads on top of each other
    (dict(o_stride_head=128, o_stride_token=128), 7),            # head h+1 = token n+1
    (dict(batch=2, o_stride_batch=256, o_stride_head=128, o_stride_token=256), 7),
])
def test_layout_validation(lib, kw, code):
    d = desc(**kw)
    assert lib.losa_dense_attn(d, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == code
    assert lib.losa_sparse_attn(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == code
    assert lib.losa_dense_attn_mass_workspace(d) == -1


@pytest.mark.parametrize("kw", [
    # [B, N, H, D] read and written in place
    dict(batch=2, stride_batch=1000 * 2 * 128, stride_head=128, stride_token=2 * 128,
         o_stride_batch=1000 * 2 * 128, o_stride_head=128, o_stride_token=2 * 128),
    # q/k/v of a packed [B, N, 3, H, D] projection, O a [B, N, H, D] tensor
    dict(batch=2, stride_batch=3 * 1000 * 2 * 128, stride_head=128, stride_token=3 * 2 * 128,
         o_stride_batch=1000 * 2 * 128, o_stride_head=128, o_stride_token=2 * 128),
    # O a slice of a wider buffer (token stride above the packed row)
    dict(o_stride_batch=0, o_stride_head=128, o_stride_token=4 * 128),
    # a size-1 batch: its stride is never used, whatever its value
    dict(stride_batch=12, stride_head=128, stride_token=2 * 128,
         o_stride_batch=-3, o_stride_head=128, o_stride_token=2 * 128),
])
def test_layouts_accepted(lib, kw):
    # the workspace query validates the descriptor and launches nothing
    assert lib.losa_dense_attn_mass_workspace(desc(**kw)) > 0


def test_null_and_alignment(lib):
    d = desc()
    assert lib.losa_dense_attn(None, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == 1
    assert lib.losa_dense_attn(d, NULL, FAKE, FAKE, FAKE, NULL, NULL) == 1
    assert lib.losa_dense_attn(d, FAKE, FAKE, FAKE, NULL, NULL, NULL) == 1
    assert lib.losa_dense_attn(d, ODD, FAKE, FAKE, FAKE, NULL, NULL) == 5
    assert lib.losa_dense_attn(d, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10001), NULL) == 5
    assert lib.losa_sparse_attn(d, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, NULL, NULL) == 1
    assert lib.losa_sparse_attn(d, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, NULL, NULL) == 1
    assert lib.losa_sparse_attn(d, FAKE, FAKE, ODD, FAKE, FAKE, FAKE, NULL, NULL) == 5
    # block mass needs lse or a scratch buffer for the first pass
    assert lib.losa_block_mass(d, FAKE, FAKE, NULL, NULL, FAKE, NULL) == 1
    assert lib.losa_block_mass(d, FAKE, FAKE, FAKE, NULL, NULL, NULL) == 1
    assert lib.losa_block_mass(d, FAKE, ODD, FAKE, NULL, FAKE, NULL) == 5


def test_dense_attn_mass_workspace_and_validation(lib):
    d = desc(batch=1, heads=12, seq_len=32760, block=64)
    need = lib.losa_dense_attn_mass_workspace(d)
    # per-row block sums [B*H, nb, N] (256-byte padded) + per-row offsets [B*H, N]
    rowsum = 4 * 12 * 512 * 32760
    assert need == (rowsum + 255) // 256 * 256 + 4 * 12 * 32760
    assert lib.losa_dense_attn_mass_workspace(None) == -1
    # the least it takes: one (b, h) per pass
    least = lib.losa_dense_attn_mass_workspace_min(d)
    assert least == (4 * 512 * 32760 + 255) // 256 * 256 + 4 * 32760
    assert lib.losa_dense_attn_mass_workspace_min(None) == -1
    assert lib.losa_dense_attn_mass_workspace_min(desc(head_dim=96)) == -1
    args = [FAKE, FAKE, FAKE, FAKE, NULL, FAKE]
    assert lib.losa_dense_attn_mass(d, *args, FAKE, least - 1, NULL) == 8
    assert lib.losa_dense_attn_mass(d, *args, FAKE, 0, NULL) == 8
    assert lib.losa_dense_attn_mass(d, *args, FAKE, -1, NULL) == 8
    assert lib.losa_dense_attn_mass(d, *args, NULL, need, NULL) == 1
    assert lib.losa_dense_attn_mass(d, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, need, NULL) == 1
    assert lib.losa_dense_attn_mass(d, *args, ctypes.c_void_p(0x10010), need, NULL) == 5
    assert lib.losa_dense_attn_mass(d, FAKE, FAKE, ODD, FAKE, NULL, FAKE, FAKE, need, NULL) == 5


@pytest.mark.parametrize("rows,nkb,tau,code", [
    (0, 16, 0.99, 2), (4, 0, 0.99, 2), (4, 1025, 0.99, 2), (4, 16, 0.0, 4),
    (4, 16, -0.5, 4), (4, 16, float("nan"), 4),
])
def test_select_validation(lib, rows, nkb, tau, code):
    assert lib.losa_select(rows, nkb, FAKE, tau, FAKE, FAKE, NULL) == code


def test_select_null_and_alignment(lib):
    assert lib.losa_select(4, 16, NULL, 0.99, FAKE, FAKE, NULL) == 1
    assert lib.losa_select(4, 16, FAKE, 0.99, NULL, FAKE, NULL) == 1
    assert lib.losa_select(4, 16, FAKE, 0.99, FAKE, NULL, NULL) == 1
    assert lib.losa_select(4, 16, ctypes.c_void_p(0x10001), 0.99, FAKE, FAKE, NULL) == 5


def test_per_row_select_mask_and_retained_validation(lib):
    d = desc()
    assert lib.losa_select_per_row(4, 16, FAKE, NULL, 1, FAKE, FAKE, NULL) == 1
    assert lib.losa_select_per_row(4, 16, FAKE, FAKE, 0, FAKE, FAKE, NULL) == 7
    assert lib.losa_select_per_row(0, 16, FAKE, FAKE, 1, FAKE, FAKE, NULL) == 2
    assert lib.losa_select_per_row(4, 1025, FAKE, FAKE, 1, FAKE, FAKE, NULL) == 2
    assert lib.losa_select_per_row(4, 16, FAKE, ctypes.c_void_p(0x10004), 1, FAKE, FAKE,
                                   NULL) == 5
    assert lib.losa_block_mask(4, 16, NULL, FAKE, FAKE, NULL) == 1
    assert lib.losa_block_mask(4, 16, FAKE, FAKE, NULL, NULL) == 1
    assert lib.losa_block_mask(4, 0, FAKE, FAKE, FAKE, NULL) == 2
    assert lib.losa_block_mask(4, 16, ctypes.c_void_p(0x10002), FAKE, FAKE, NULL) == 5
    assert lib.losa_retained_mass(None, FAKE, FAKE, FAKE, NULL) == 1
    assert lib.losa_retained_mass(d, NULL, FAKE, FAKE, NULL) == 1
    assert lib.losa_retained_mass(d, FAKE, FAKE, ctypes.c_void_p(0x10002), NULL) == 5
    assert lib.losa_retained_mass(desc(block=32), FAKE, FAKE, FAKE, NULL) == 2


def test_sparse_plan_validation(lib):
    d = desc(batch=1, heads=12, seq_len=32760, block=64)
    # a 4-word header, then one slot per 128-row work item, padded to whole
    # rounds of 8 runs (one per XCD) of 16 items
    assert lib.losa_sparse_plan_size(d) == 4 * (4 + 12 * 256)
    assert lib.losa_sparse_plan_size(desc(seq_len=118800, block=128, heads=24)) == \
        4 * (4 + 128 * ((24 * 929 + 127) // 128))
    assert lib.losa_sparse_plan_size(desc(batch=2, heads=48, seq_len=17776, head_dim=64)) \
        == 4 * (4 + 128 * ((2 * 48 * 139 + 127) // 128))
    assert lib.losa_sparse_plan_size(None) == -1
    need = lib.losa_sparse_plan_size(d)
    assert lib.losa_sparse_plan(d, NULL, FAKE, need, NULL) == 1
    assert lib.losa_sparse_plan(d, FAKE, NULL, need, NULL) == 1
    assert lib.losa_sparse_plan(d, FAKE, ctypes.c_void_p(0x10002), need, NULL) == 5
    assert lib.losa_sparse_plan(d, FAKE, FAKE, need - 4, NULL) == 8
    assert lib.losa_sparse_plan(desc(block=32), FAKE, FAKE, need, NULL) == 2
    args = [FAKE, FAKE, FAKE, FAKE, FAKE]
    assert lib.losa_sparse_attn_planned(d, *args, NULL, need, FAKE, NULL, NULL) == 1
    assert lib.losa_sparse_attn_planned(d, *args, ctypes.c_void_p(0x10002), need, FAKE, NULL,
                                        NULL) == 5
    assert lib.losa_sparse_attn_planned(d, *args, FAKE, need, NULL, NULL, NULL) == 1
    assert lib.losa_sparse_attn_planned(desc(head_dim=96), *args, FAKE, need, FAKE, NULL,
                                        NULL) == 2
    # a plan shorter than the shape's plan size is refused before any launch
    assert lib.losa_sparse_attn_planned(d, *args, FAKE, need - 4, FAKE, NULL, NULL) == 8
    assert lib.losa_sparse_attn_planned(d, *args, FAKE, 0, FAKE, NULL, NULL) == 8


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.LosaLibraryMissing):
        _lib.load(str(tmp_path / "missing.so"))


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """The no-allocation mass entry takes B*H*N <= LOSA_NOALLOC_MAX_ROWS and
    refuses larger inputs on the host, before touching the device."""
    assert _lib.NOALLOC_MAX_ROWS == 4194304
    big = desc(batch=1, heads=65, seq_len=65536, head_dim=64, block=64)   # 4 259 840 rows
    assert lib.losa_block_mass_noalloc(big, FAKE, FAKE, FAKE, NULL) == 9
    assert lib.losa_block_mass_noalloc(desc(head_dim=96), FAKE, FAKE, FAKE, NULL) == 2
    assert lib.losa_block_mass_noalloc(None, FAKE, FAKE, FAKE, NULL) == 1
    assert lib.losa_block_mass_noalloc(desc(), FAKE, NULL, FAKE, NULL) == 1
    assert lib.losa_block_mass_noalloc(desc(), FAKE, FAKE, NULL, NULL) == 1
