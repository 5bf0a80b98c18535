"""float64 oracle of chunked prefill attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy, float64,
no blocking beyond a row loop that bounds memory, no reordering of the
definition.  Shares no code with the HIP library.

Notation (from the pages' problem statement):
  R   chunk rows (query tokens of this chunk, at absolute positions H .. H+R-1)
  H   history length (tokens already in the cache before the chunk)
  Hq  query heads, Hkv key/value heads, G = Hq / Hkv (grouped-query heads)
  d   head dimension, ps page size (tokens per page)
  ctx = H + R, the tokens the block table covers (the chunk's own K/V are
  already written into its pages).

Layouts:
  q       [R][Hq][d]
  k_pages [n_pool_pages][ps][Hkv][d]  (likewise v_pages)
  block_table[j] = pool page holding logical page j
  k, v    [>= ctx][Hkv][d]            (contiguous KV)
  out     [R][Hq][d]
"""

import math

import numpy as np


def decode_f16(raw):
    """IEEE binary16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(raw, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_bf16(raw):
    """bfloat16 bit patterns (uint16) -> float64, exactly: a bfloat16 is the
    upper half of a binary32."""
    wide = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def gather_pages(pages, block_table, n_tokens, page_size):
    """Contiguous [n_tokens][Hkv][d] from paged storage.

    Logical token j lives in slot j mod ps of pool page block_table[j div ps]
    (the paged KV cache of the issue "Metal: paged-KV prefill is 4.43x slower
    than contiguous KV at 32K": fixed-size pages addressed through a block
    table).  Slots past n_tokens are never read.
    """
    pages = np.asarray(pages)
    block_table = np.asarray(block_table)
    out = np.empty((n_tokens,) + pages.shape[2:], dtype=pages.dtype)
    for j in range(n_tokens):
        pool_page = block_table[j // page_size]
        out[j] = pages[pool_page, j % page_size]
    return out


def _row_block(n_query_vectors_per_row, n_keys, budget=1 << 24):
    return max(1, budget // max(1, n_query_vectors_per_row * n_keys))


def causal_attention_rows(q, k, v, history_len, rows):
    """Output rows ``rows`` of causal attention of the chunk against K/V.

    Chunk row i sits at absolute position H + i and sees keys 0 .. H + i
    inclusive: all of the history plus the chunk's own tokens up to and
    including itself.  Query head h reads KV head h div G.  The scale is
    1/sqrt(d).  Returns [len(rows)][Hq][d] in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    n_q_heads, d = q.shape[1], q.shape[2]
    n_kv_heads = k.shape[1]
    group = n_q_heads // n_kv_heads
    scale = 1.0 / math.sqrt(d)
    out = np.empty((len(rows), n_q_heads, d), dtype=np.float64)
    if len(rows) == 0:
        return out
    block = _row_block(group, history_len + int(rows.max()) + 1)
    for g in range(n_kv_heads):
        heads = slice(g * group, (g + 1) * group)
        for b in range(0, len(rows), block):
            rb = rows[b:b + block]
            n_keys = history_len + int(rb.max()) + 1
            qb = q[rb, heads, :].reshape(len(rb) * group, d)
            scores = (qb @ k[:n_keys, g, :].T) * scale
            last_visible = history_len + np.repeat(rb, group)
            visible = np.arange(n_keys)[None, :] <= last_visible[:, None]
            scores = np.where(visible, scores, -np.inf)
            scores = scores - scores.max(axis=1, keepdims=True)
            weights = np.exp(scores)
            weights = weights / weights.sum(axis=1, keepdims=True)
            out[b:b + len(rb), heads, :] = (weights @ v[:n_keys, g, :]).reshape(len(rb), group, d)
    return out


def causal_attention(q, k, v, history_len):
    """softmax(Q K^T / sqrt(d)) V over contiguous K/V, every chunk row."""
    return causal_attention_rows(q, k, v, history_len, np.arange(np.asarray(q).shape[0]))


def paged_causal_attention(q, k_pages, v_pages, block_table, history_len, page_size):
    """The paged entry point: gather the ctx = H + R tokens through the block
    table, then the same computation as over contiguous K/V."""
    ctx = history_len + np.asarray(q).shape[0]
    k = gather_pages(k_pages, block_table, ctx, page_size)
    v = gather_pages(v_pages, block_table, ctx, page_size)
    return causal_attention(q, k, v, history_len)


def page_aligned_split_ranges(ctx, page_size, n_splits):
    """Cut the logical key axis [0, ctx) into n_splits contiguous ranges of
    ceil(pages / S) pages each (the last takes the remainder; trailing ranges
    may be empty).  S is clamped to the number of pages.  This is the reading
    of the PR's "history split" that the oracle uses; any partition gives the
    same merged result."""
    n_pages = -(-ctx // page_size)
    n_splits = max(1, min(n_splits, n_pages))
    per = -(-n_pages // n_splits)
    ranges = []
    for s in range(n_splits):
        start = min(s * per * page_size, ctx)
        end = min((s + 1) * per * page_size, ctx)
        ranges.append((start, end))
    return ranges


def split_partials(q, k, v, history_len, ranges):
    """Per-range partial attention.

    For range s = [a, b) and query vector (row i, head h) the visible keys are
    j in [a, b) with j <= H + i.  Returns O [S][R][Hq][d] (the range's own
    softmax-weighted mean of V) and lse [S][R][Hq] = m + ln(l) with m the
    range's max score and l = sum exp(score - m); a range with no visible key
    has O = 0 and lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_rows, n_q_heads, d = q.shape
    n_kv_heads = k.shape[1]
    group = n_q_heads // n_kv_heads
    scale = 1.0 / math.sqrt(d)
    n_splits = len(ranges)
    o_part = np.zeros((n_splits, n_rows, n_q_heads, d), dtype=np.float64)
    lse = np.full((n_splits, n_rows, n_q_heads), -np.inf, dtype=np.float64)
    rows = np.arange(n_rows)
    for s, (a, b) in enumerate(ranges):
        if b <= a:
            continue
        for g in range(n_kv_heads):
            heads = slice(g * group, (g + 1) * group)
            qg = q[:, heads, :].reshape(n_rows * group, d)
            scores = (qg @ k[a:b, g, :].T) * scale
            last_visible = history_len + np.repeat(rows, group)
            visible = np.arange(a, b)[None, :] <= last_visible[:, None]
            any_visible = visible.any(axis=1)
            scores = np.where(visible, scores, -np.inf)
            m = np.where(any_visible, scores.max(axis=1), 0.0)
            weights = np.where(visible, np.exp(scores - m[:, None]), 0.0)
            l = weights.sum(axis=1)
            safe_l = np.where(any_visible, l, 1.0)
            o = (weights @ v[a:b, g, :]) / safe_l[:, None]
            o_part[s, :, heads, :] = o.reshape(n_rows, group, d)
            lse_g = np.where(any_visible, m + np.log(safe_l), -np.inf)
            lse[s, :, heads] = lse_g.reshape(n_rows, group)
    return o_part, lse


def merge_partials(o_part, lse):
    """Log-sum-exp merge of split partials: L = logsumexp_s(lse_s),
    out = sum_s exp(lse_s - L) O_s.  Ranges with lse = -inf weigh 0.  Every
    query vector must have at least one range with a visible key."""
    o_part = np.asarray(o_part, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    top = lse.max(axis=0)
    total = np.log(np.exp(lse - top[None]).sum(axis=0)) + top
    weights = np.exp(lse - total[None])
    return (weights[..., None] * o_part).sum(axis=0)


def split_causal_attention(q, k, v, history_len, ranges):
    """Split form of ``causal_attention``: partials per range, then the merge."""
    o_part, lse = split_partials(q, k, v, history_len, ranges)
    return merge_partials(o_part, lse)
