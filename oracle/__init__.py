"""fp64 CPU oracle for the LoSA attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing here is part of the product: only the test
suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library and does
not import the ``block_sparse_attention_losa_amd`` package.

Sources (the pages describing LoSA, arXiv 2608.12032):
  * "Abstract (arXiv)" on the mlsanity.com paper index page,
  * "Summary & Methodology Analysis" and FAQ Q4-Q6 on the legiblepapers page,
  * "What the Researchers Propose" and "How It Works in Practice"
    (Phases 1-3) on the ubos.tech blog post,
  * "Abstract Summary" and "Key Highlights" on the aitobox blog post,
  * "Key Findings" and "What Comes Next" on the ubos.tech blog post.
"""

from .losa_oracle import (  # noqa: F401
    num_blocks,
    block_rows,
    dense_attention,
    row_lse,
    block_mass,
    select_row,
    select,
    sparse_attention,
    kept_key_mask,
    retained_mass,
    select_rows,
    block_mask,
)
