"""Oracle of the KV append: writing a chunk's K and V rows into their pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy, one
token at a time, no reordering.  Shares no code with the HIP library.

The issue "Metal: paged-KV prefill is 4.43x slower than contiguous KV at 32K"
(the closing "Expected vs actual" notes) names publishing completed KV pages
as the step after a prefill chunk; the attention of that chunk reads its own
K/V from the pages (the cache holds ctx = H + R tokens when the attention
runs).  The append is that write: chunk row i is the token at absolute
position H + i, stored in slot (H + i) mod ps of pool page
block_table[(H + i) div ps], one [Hkv][d] row per token for K and for V.
Nothing else in the pool changes.  It moves raw 16-bit patterns: no
arithmetic, so the result is exact.
"""

import numpy as np


def kv_append(k_pages, v_pages, block_table, history_len, page_size, k_new, v_new):
    """The pools after appending k_new/v_new [R][Hkv][d] at positions H .. H+R-1.

    k_pages, v_pages: [n_pool_pages][ps][Hkv][d] (any element type, copied
    bit for bit).  Returns new arrays; the inputs are left unchanged.
    """
    k_out = np.array(k_pages, copy=True)
    v_out = np.array(v_pages, copy=True)
    block_table = np.asarray(block_table)
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    assert k_new.shape == v_new.shape and k_new.shape[1:] == k_out.shape[2:]
    for i in range(k_new.shape[0]):
        pos = history_len + i
        pool_page = block_table[pos // page_size]
        slot = pos % page_size
        k_out[pool_page, slot] = k_new[i]
        v_out[pool_page, slot] = v_new[i]
    return k_out, v_out
