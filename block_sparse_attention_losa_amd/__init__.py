"""LoSA attention hot path on MI355X (gfx950): dense attention, block mass
map, threshold selection and block-sparse attention over frozen block lists,
as hand-written HIP kernels behind the C-ABI of ``include/losa.h``.

The functions below are argument marshalling around ``liblosa.so``; they
raise if the library has not been built (``python -m
block_sparse_attention_losa_amd.build``).
"""

from ._lib import LosaError, LosaLibraryMissing  # noqa: F401
from .frozen import FrozenLists  # noqa: F401
from .api import (block_mask, block_mass, block_mass_noalloc, dense_attn,  # noqa: F401
                  dense_attn_mass, dense_attn_mass_workspace_bytes, num_blocks,
                  retained_mass, select, select_per_row, sparse_attn, sparse_plan)

__all__ = ["dense_attn", "block_mass", "block_mass_noalloc", "dense_attn_mass", "dense_attn_mass_workspace_bytes",
           "select", "select_per_row", "sparse_attn", "sparse_plan", "block_mask",
           "retained_mass",
           "num_blocks", "FrozenLists", "LosaError", "LosaLibraryMissing"]
