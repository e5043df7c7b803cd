"""Paged KV-cache gather (test infrastructure only).

Declarative Attention post, "Declarative attention protocol": the serving
engine keeps the KV cache in fixed-size blocks (pages) of usually 16-32
tokens, and attention kernels read whole blocks.  Layout read here:
pool[page, kv_head, slot, d], token j of a sequence lives in page
page_table[j // P] at slot j % P.
"""

import numpy as np


def gather_pages(pool, page_table, seq_len, g):
    """Contiguous [seq_len, D] keys (or values) of one sequence and KV head g,
    by plain fancy indexing through the page table."""
    pool = np.asarray(pool)
    P = pool.shape[2]
    j = np.arange(int(seq_len))
    pages = np.asarray(page_table, dtype=np.int64)[j // P]
    return np.asarray(pool[pages, g, j % P], dtype=np.float64)
