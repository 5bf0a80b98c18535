"""Oracle of multi-sequence (varlen) chunked prefill over one shared page pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy, float64,
one sequence at a time.  Shares no code with the HIP library.

The issue "Metal: paged-KV prefill is 4.43x slower than contiguous KV at 32K"
(its opening problem statement) places paged KV in serving with continuous
batching and prefix caching: several sequences, each with its own history
and its own pages, are prefilled together.  Here a batch of n sequences
shares one K/V page pool.  Sequence s has

  * history length H_s (tokens already in its cache),
  * R_s chunk rows: rows cu_rows[s] .. cu_rows[s+1]-1 of the packed q and
    out, at positions H_s .. H_s + R_s - 1 of that sequence,
  * its own block table, row s of block_tables: logical page j of the
    sequence lives in pool page block_tables[s][j].

Each sequence's rows are exactly the single-sequence paged attention of those
rows over its own ctx_s = H_s + R_s tokens: sequences never see each other's
keys, and pool pages that several tables name (a shared prefix) are read by
each of them.  Rows that belong to no sequence are not defined; this oracle
leaves them 0.
"""

import numpy as np

from oracle.attention import causal_attention, gather_pages


def varlen_paged_attention(q, k_pages, v_pages, block_tables, cu_rows, history_lens, page_size):
    """out [total_rows][Hq][d] float64 for a packed batch of sequences.

    q: [total_rows][Hq][d]; k_pages, v_pages: [n_pool][ps][Hkv][d];
    block_tables: [n][>= max ceil(ctx_s / ps)]; cu_rows: [n + 1]
    non-decreasing row offsets; history_lens: [n].
    """
    q = np.asarray(q, dtype=np.float64)
    block_tables = np.asarray(block_tables)
    cu_rows = np.asarray(cu_rows, dtype=np.int64)
    history_lens = np.asarray(history_lens, dtype=np.int64)
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(len(history_lens)):
        r0, r1 = int(cu_rows[s]), int(cu_rows[s + 1])
        if r1 == r0:
            continue
        hist = int(history_lens[s])
        ctx = hist + (r1 - r0)
        k = gather_pages(k_pages, block_tables[s], ctx, page_size)
        v = gather_pages(v_pages, block_tables[s], ctx, page_size)
        out[r0:r1] = causal_attention(q[r0:r1], k, v, hist)
    return out
