"""The PR's host rules, transcribed from its prose (TEST INFRASTRUCTURE ONLY).

Source: PR "perf: scale prefill attention splits with GPU cores on Apple7/8",
section "What changed" and the explanatory note after "Testing".  Both are
pinned in ``tests/test_oracle_pins.py`` by the split table and the piece sizes
the PR prints (``tests/golden/``).
"""


def page_split_rule(gpu_cores, kv_heads, tiles, per_core=32, floor=32, slot_cap=256, max_splits=32):
    """Splits of the history for one prefill piece on the register tile.

    The PR aims at ``per_core`` threadgroups per GPU core, with at least
    ``floor`` and at most ``slot_cap`` threadgroups per KV head (the cap is
    the number of tile slots a full 2048-row chunk already uses), divides by
    the piece's row tiles and clamps the quotient to 1 .. ``max_splits``.
    All divisions are integer divisions.
    """
    per_head = min(slot_cap, max(floor, (per_core * gpu_cores) // kv_heads))
    return min(max(per_head // tiles, 1), max_splits)


def page_piece_rows(history_len, chunk_rows=2048, budget=1 << 25):
    """Rows per prefill piece: halve the chunk until rows * (history + rows)
    fits the budget of 2^25 (the PR's display-latency guard)."""
    rows = chunk_rows
    while rows > 1 and rows * (history_len + rows) > budget:
        rows //= 2
    return rows
