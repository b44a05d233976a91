"""Thin torch-facing binding of the C-ABI (same names as the C entry points).

Only argument marshalling happens here: output tensors are allocated with
``torch.empty`` on the inputs' device and every computation runs in the HIP
kernels of ``liblosa.so``, enqueued on torch's current stream.
"""

import ctypes
import math

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.LOSA_BF16, torch.float32: _lib.LOSA_FP32}


def num_blocks(seq_len: int, block: int) -> int:
    return (int(seq_len) + int(block) - 1) // int(block)


def _layout(t):
    """Element strides (batch, head, token) of a [B, H, N, D]-shaped tensor,
    or zeros when it is contiguous.  Non-contiguous views (e.g. a
    [B, N, H, D] tensor permuted to [B, H, N, D], or one of q/k/v of a packed
    projection) need a contiguous head dim and bfloat16."""
    if t is None or t.is_contiguous():
        return (0, 0, 0)
    if t.stride(-1) != 1:
        raise ValueError("the head dimension must be contiguous")
    if t.dtype != torch.bfloat16:
        raise TypeError("strided layouts are supported for bfloat16 only")
    return (t.stride(0), t.stride(1), t.stride(2))


def make_desc(q: torch.Tensor, block: int, scale=None, k=None, v=None, o=None) -> _lib.AttnDesc:
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, D] tensors")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    b, h, n, d = q.shape
    lay = _layout(q)
    for t in (k, v):
        if t is not None and _layout(t) != lay:
            raise ValueError("q, k and v must share one memory layout")
    return _lib.AttnDesc(b, h, n, d, int(block), _DTYPES[q.dtype],
                         0.0 if scale is None else float(scale), *lay, *_layout(o))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_inputs(*ts, strided=()):
    """Device checks; tensors in ``strided`` may be non-contiguous views
    (their layout goes to the descriptor), the others must be contiguous."""
    present = [t for t in tuple(strided) + tuple(ts) if t is not None]
    for t in present:
        if not t.is_cuda:
            raise ValueError("tensors must live on a GPU")
        if t.device != present[0].device:
            raise ValueError("tensors must share one device")
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_out(t, shape, dtype, name):
    """A caller-supplied output must have the exact shape and dtype the
    kernel writes: the C entry points take raw pointers and cannot see a
    short buffer."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def dense_attn(q, k, v, block: int = 64, scale=None, o=None, lse=None, want_lse=True):
    """Dense softmax attention; returns ``(o, lse)`` (lse None if not wanted).
    q, k, v (and o) are [B, H, N, D]; bfloat16 views with other strides (a
    permuted [B, N, H, D] tensor, slices of a packed projection) are read
    and written in place."""
    _check_inputs(lse, strided=(q, k, v, o))
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    _check_out(o, q.shape, q.dtype, "o")
    _check_out(lse, q.shape[:3], torch.float32, "lse")
    if o is None:
        o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    desc = make_desc(q, block, scale, k, v, o)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    lib = _lib.load()
    _lib.check("losa_dense_attn", lib.losa_dense_attn(
        desc, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(q)))
    return o, lse


def block_mass(q, k, block: int = 64, lse=None, scale=None, mass=None, lse_scratch=None):
    """Block mass map ``[B, H, nb, nb]`` (float32); runs the lse pass first
    when ``lse`` is None."""
    _check_inputs(mass, lse, lse_scratch, strided=(q, k))
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q, k must share shape and dtype")
    desc = make_desc(q, block, scale, k)
    b, h, n, _ = q.shape
    nb = num_blocks(n, block)
    _check_out(mass, (b, h, nb, nb), torch.float32, "mass")
    _check_out(lse, (b, h, n), torch.float32, "lse")
    _check_out(lse_scratch, (b, h, n), torch.float32, "lse_scratch")
    if mass is None:
        mass = torch.empty((b, h, nb, nb), dtype=torch.float32, device=q.device)
    if lse is None and lse_scratch is None:
        lse_scratch = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    _lib.check("losa_block_mass", lib.losa_block_mass(
        desc, _ptr(q), _ptr(k), _ptr(lse), _ptr(lse_scratch), _ptr(mass), _stream(q)))
    return mass


def block_mass_noalloc(q, k, block: int = 64, scale=None, mass=None):
    """Two-pass block mass map whose first pass keeps its lse in the
    library's static scratch, so the library allocates no device memory
    (pass ``mass`` to allocate nothing here either).  B*H*N must not exceed
    ``NOALLOC_MAX_ROWS``; calls overlapping on one GPU race on the scratch."""
    _check_inputs(mass, strided=(q, k))
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q, k must share shape and dtype")
    desc = make_desc(q, block, scale, k)
    b, h, n, _ = q.shape
    nb = num_blocks(n, block)
    _check_out(mass, (b, h, nb, nb), torch.float32, "mass")
    if mass is None:
        mass = torch.empty((b, h, nb, nb), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    _lib.check("losa_block_mass_noalloc", lib.losa_block_mass_noalloc(
        desc, _ptr(q), _ptr(k), _ptr(mass), _stream(q)))
    return mass


def dense_attn_mass_workspace_bytes(q, block: int = 64, minimum: bool = False) -> int:
    """Workspace bytes :func:`dense_attn_mass` needs for inputs shaped like q
    to run every (b, h) in one pass, or with ``minimum`` the least it takes
    (one (b, h) per pass)."""
    lib = _lib.load()
    fn = lib.losa_dense_attn_mass_workspace_min if minimum else lib.losa_dense_attn_mass_workspace
    n = fn(make_desc(q, block))
    if n < 0:
        raise ValueError("unsupported shape for dense_attn_mass")
    return int(n)


def dense_attn_mass(q, k, v, block: int = 64, scale=None, o=None, lse=None, mass=None,
                    workspace=None, want_lse=True, max_workspace_bytes=None):
    """Construction step in one sweep: dense attention and the block mass map
    of the same inputs.  Returns ``(o, lse, mass)``.  ``workspace`` is a
    uint8 device tensor of at least ``dense_attn_mass_workspace_bytes(q,
    block, minimum=True)`` bytes; the call makes as few passes over the
    heads as its size allows.  When None, one is allocated here: the full
    size, or at most ``max_workspace_bytes`` (but never below the minimum).
    The results do not depend on the workspace size."""
    _check_inputs(lse, mass, workspace, strided=(q, k, v, o))
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    b, h, n, _ = q.shape
    nb = num_blocks(n, block)
    _check_out(o, q.shape, q.dtype, "o")
    _check_out(lse, (b, h, n), torch.float32, "lse")
    _check_out(mass, (b, h, nb, nb), torch.float32, "mass")
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    if o is None:
        o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    desc = make_desc(q, block, scale, k, v, o)
    if lse is None and want_lse:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if mass is None:
        mass = torch.empty((b, h, nb, nb), dtype=torch.float32, device=q.device)
    if workspace is None:
        size = dense_attn_mass_workspace_bytes(q, block)
        if max_workspace_bytes is not None:
            size = max(min(size, int(max_workspace_bytes)),
                       dense_attn_mass_workspace_bytes(q, block, minimum=True))
        workspace = torch.empty(size, dtype=torch.uint8, device=q.device)
    lib = _lib.load()
    _lib.check("losa_dense_attn_mass", lib.losa_dense_attn_mass(
        desc, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(mass), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))
    return o, lse, mass


def select(mass, threshold: float = 0.99, idx=None, count=None):
    """Threshold selection over the last axis of ``mass``; returns
    ``(idx, count)`` with idx shaped like mass (int32; entries at and past
    count are left as allocated) and count shaped ``mass.shape[:-1]``."""
    _check_inputs(mass, idx, count)
    if mass.dtype != torch.float32:
        raise TypeError("mass must be float32")
    nkb = mass.shape[-1]
    rows = mass.numel() // nkb if nkb else 0
    _check_out(idx, mass.shape, torch.int32, "idx")
    _check_out(count, mass.shape[:-1], torch.int32, "count")
    if idx is None:
        idx = torch.empty(mass.shape, dtype=torch.int32, device=mass.device)
    if count is None:
        count = torch.empty(mass.shape[:-1], dtype=torch.int32, device=mass.device)
    lib = _lib.load()
    _lib.check("losa_select", lib.losa_select(
        rows, nkb, _ptr(mass), float(threshold), _ptr(idx), _ptr(count), _stream(mass)))
    return idx, count


def select_per_row(mass, thresholds, rows_per_threshold: int = 1, idx=None, count=None):
    """Threshold selection with a threshold per group of ``rows_per_threshold``
    rows of ``mass`` (flattened over its leading axes); ``thresholds`` is a
    float64 device tensor of ``ceil(rows / rows_per_threshold)`` values.
    Returns ``(idx, count)`` as :func:`select`."""
    _check_inputs(mass, thresholds, idx, count)
    if mass.dtype != torch.float32 or thresholds.dtype != torch.float64:
        raise TypeError("mass must be float32 and thresholds float64")
    nkb = mass.shape[-1]
    rows = mass.numel() // nkb if nkb else 0
    if thresholds.numel() < (rows + rows_per_threshold - 1) // max(1, rows_per_threshold):
        raise ValueError("too few thresholds for the rows")
    _check_out(idx, mass.shape, torch.int32, "idx")
    _check_out(count, mass.shape[:-1], torch.int32, "count")
    if idx is None:
        idx = torch.empty(mass.shape, dtype=torch.int32, device=mass.device)
    if count is None:
        count = torch.empty(mass.shape[:-1], dtype=torch.int32, device=mass.device)
    lib = _lib.load()
    _lib.check("losa_select_per_row", lib.losa_select_per_row(
        rows, nkb, _ptr(mass), _ptr(thresholds), int(rows_per_threshold), _ptr(idx),
        _ptr(count), _stream(mass)))
    return idx, count


def block_mask(idx, count, mask=None):
    """The lists as a uint8 mask shaped like ``idx`` (1 = key block kept)."""
    _check_inputs(idx, count, mask)
    if idx.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("idx and count must be int32")
    nkb = idx.shape[-1]
    rows = idx.numel() // nkb if nkb else 0
    if count.numel() != rows:
        raise ValueError("count must have one entry per row of idx")
    _check_out(mask, idx.shape, torch.uint8, "mask")
    if mask is None:
        mask = torch.empty(idx.shape, dtype=torch.uint8, device=idx.device)
    lib = _lib.load()
    _lib.check("losa_block_mask", lib.losa_block_mask(
        rows, nkb, _ptr(idx), _ptr(count), _ptr(mask), _stream(idx)))
    return mask


def retained_mass(lse_kept, lse_dense, block: int = 64, head_dim: int = 128, retained=None):
    """Drift diagnostic: per query block, the share of the dense attention
    mass that the frozen lists cover, from the lse of a sparse pass and of a
    dense pass on the same inputs (both ``[B, H, N]`` float32).  Returns
    ``[B, H, nb]`` float32."""
    _check_inputs(lse_kept, lse_dense, retained)
    if lse_kept.shape != lse_dense.shape or lse_kept.dim() != 3:
        raise ValueError("expected two [B, H, N] lse tensors")
    if lse_kept.dtype != torch.float32 or lse_dense.dtype != torch.float32:
        raise TypeError("lse tensors must be float32")
    b, h, n = lse_kept.shape
    nb = num_blocks(n, block)
    desc = _lib.AttnDesc(b, h, n, int(head_dim), int(block), _lib.LOSA_BF16, 0.0)
    _check_out(retained, (b, h, nb), torch.float32, "retained")
    if retained is None:
        retained = torch.empty((b, h, nb), dtype=torch.float32, device=lse_kept.device)
    lib = _lib.load()
    _lib.check("losa_retained_mass", lib.losa_retained_mass(
        desc, _ptr(lse_kept), _ptr(lse_dense), _ptr(retained), _stream(lse_kept)))
    return retained


def sparse_plan(count, block: int = 64, head_dim: int = 128, plan=None):
    """Launch plan for :func:`sparse_attn` over lists with these counts
    (``[B, H, nb]`` int32): the work items longest-first.  Made once per set
    of frozen lists; returns an int32 device tensor."""
    _check_inputs(count)
    if count.dtype != torch.int32 or count.dim() != 3:
        raise TypeError("count must be an int32 [B, H, nb] tensor")
    b, h, nb = count.shape
    desc = _lib.AttnDesc(b, h, nb * int(block), int(head_dim), int(block), _lib.LOSA_BF16, 0.0)
    lib = _lib.load()
    size = lib.losa_sparse_plan_size(desc)
    if size < 0:
        raise ValueError("unsupported shape for sparse_plan")
    if plan is None:
        plan = torch.empty(size // 4, dtype=torch.int32, device=count.device)
    elif plan.dtype != torch.int32 or not plan.is_contiguous():
        raise TypeError("plan must be a contiguous int32 tensor")
    _lib.check("losa_sparse_plan", lib.losa_sparse_plan(
        desc, _ptr(count), _ptr(plan), plan.numel() * 4, _stream(count)))
    return plan


def sparse_attn(q, k, v, idx, count, block: int = 64, scale=None, o=None, lse=None,
                want_lse=False, plan=None):
    """Block-sparse attention over frozen lists; returns ``(o, lse)``.  With
    ``plan`` (from :func:`sparse_plan` on the same counts) the work runs in
    the plan's order; the results are the same."""
    _check_inputs(idx, count, lse, plan, strided=(q, k, v, o))
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    b, h, n, _ = q.shape
    nb = num_blocks(n, block)
    if tuple(idx.shape) != (b, h, nb, nb) or tuple(count.shape) != (b, h, nb):
        raise ValueError("idx must be [B,H,nb,nb] and count [B,H,nb]")
    if idx.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("idx and count must be int32")
    _check_out(o, q.shape, q.dtype, "o")
    _check_out(lse, (b, h, n), torch.float32, "lse")
    if o is None:
        o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    desc = make_desc(q, block, scale, k, v, o)
    if lse is None and want_lse:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    if plan is not None:
        if plan.dtype != torch.int32 or not plan.is_contiguous():
            raise TypeError("plan must be a contiguous int32 tensor")
        # the kernel reads one plan entry per launched workgroup
        if plan.numel() * 4 < lib.losa_sparse_plan_size(desc):
            raise ValueError("plan is smaller than sparse_plan makes for these shapes")
        _lib.check("losa_sparse_attn_planned", lib.losa_sparse_attn_planned(
            desc, _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(count), _ptr(plan),
            plan.numel() * 4, _ptr(o), _ptr(lse), _stream(q)))
        return o, lse
    _lib.check("losa_sparse_attn", lib.losa_sparse_attn(
        desc, _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(count), _ptr(o), _ptr(lse),
        _stream(q)))
    return o, lse


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
