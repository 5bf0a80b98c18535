"""Checks that pin the oracle to facts other than itself.

Each ``pin_*`` takes an oracle module (the real one, or a mutated copy in
``test_oracle_mutants.py``) and raises AssertionError when the oracle
disagrees with brute force, a closed form, torch's CPU attention with an
explicit causal mask, an invariant of the definition, or a value the pages
print.  Inputs are float64 so that only the oracle's arithmetic is on trial.
"""

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- inputs
def paged_inputs(rng, rows, history, n_q_heads, n_kv_heads, d, ps, extra_pool=3, scale=1.0):
    """float64 paged inputs with a permuted block table; unused pool pages and
    page tails are NaN, so reading them poisons the result."""
    ctx = history + rows
    n_pages = -(-ctx // ps)
    q = rng.standard_normal((rows, n_q_heads, d)) * scale
    k = rng.standard_normal((ctx, n_kv_heads, d)) * scale
    v = rng.standard_normal((ctx, n_kv_heads, d)) * scale
    pool = n_pages + extra_pool
    bt = rng.permutation(pool)[:n_pages].astype(np.int32)
    k_pages = np.full((pool, ps, n_kv_heads, d), np.nan)
    v_pages = np.full((pool, ps, n_kv_heads, d), np.nan)
    for j in range(ctx):
        k_pages[bt[j // ps], j % ps] = k[j]
        v_pages[bt[j // ps], j % ps] = v[j]
    return q, k, v, k_pages, v_pages, bt


def brute_force(q, k_pages, v_pages, bt, history, ps):
    """Definition written out with Python loops and math.fsum: no max
    subtraction, no vector ops, per-token page lookup."""
    rows, n_q_heads, d = q.shape
    n_kv_heads = k_pages.shape[2]
    group = n_q_heads // n_kv_heads
    out = np.zeros((rows, n_q_heads, d))
    for i in range(rows):
        for h in range(n_q_heads):
            g = h // group
            keys = list(range(history + i + 1))
            kv = [(k_pages[bt[j // ps], j % ps, g], v_pages[bt[j // ps], j % ps, g]) for j in keys]
            e = [math.exp(math.fsum(float(q[i, h, t]) * float(kj[t]) for t in range(d)) / math.sqrt(d))
                 for kj, _ in kv]
            z = math.fsum(e)
            for c in range(d):
                out[i, h, c] = math.fsum(ej * float(vj[c]) for ej, (_, vj) in zip(e, kv)) / z
    return out


BRUTE_SHAPES = [
    # rows, history, Hq, Hkv, d, ps
    (5, 11, 2, 1, 4, 2),
    (8, 40, 4, 2, 8, 4),
    (3, 0, 3, 1, 5, 4),
    (7, 13, 6, 3, 3, 2),
]


def max_rel(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- pins
def pin_decoders(orc):
    """Bit patterns with known values (IEEE binary16 and bfloat16 encodings),
    plus torch's own bfloat16/float16 conversion of random patterns."""
    import torch
    f16 = np.array([0x3C00, 0xC000, 0x7BFF, 0x0001, 0x3555, 0x0000, 0x8000], dtype=np.uint16)
    f16_val = [1.0, -2.0, 65504.0, 2.0 ** -24, 0.333251953125, 0.0, -0.0]
    got = orc.decode_f16(f16)
    assert np.array_equal(got, np.array(f16_val)), got
    bf = np.array([0x3F80, 0xC000, 0x7F7F, 0x3EAB, 0x0001, 0x4049], dtype=np.uint16)
    bf_val = [1.0, -2.0, 3.3895313892515355e38, 0.333984375, 2.0 ** -133, 3.140625]
    got = orc.decode_bf16(bf)
    assert np.array_equal(got, np.array(bf_val)), got
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 0x7F00, size=4096, dtype=np.uint16)  # finite positive patterns
    ref_bf = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.decode_bf16(raw), ref_bf)
    raw16 = rng.integers(0, 0x7C00, size=4096, dtype=np.uint16)
    ref_f16 = torch.from_numpy(raw16.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(orc.decode_f16(raw16), ref_f16)


def pin_gather(orc):
    """Gather through a permuted table equals the logical token order; the
    NaN-poisoned slots are never read."""
    rng = np.random.default_rng(11)
    for rows, history, hq, hkv, d, ps in BRUTE_SHAPES:
        q, k, v, kp, vp, bt = paged_inputs(rng, rows, history, hq, hkv, d, ps)
        got = orc.gather_pages(kp, bt, history + rows, ps)
        assert np.array_equal(got, k)


def pin_brute_force(orc):
    rng = np.random.default_rng(12)
    for rows, history, hq, hkv, d, ps in BRUTE_SHAPES:
        q, k, v, kp, vp, bt = paged_inputs(rng, rows, history, hq, hkv, d, ps)
        ref = brute_force(q, kp, vp, bt, history, ps)
        got = orc.paged_causal_attention(q, kp, vp, bt, history, ps)
        assert np.all(np.isfinite(got))
        assert np.max(np.abs(got - ref)) <= 1e-13, (rows, history, np.max(np.abs(got - ref)))


def pin_closed_forms(orc):
    rng = np.random.default_rng(13)
    rows, history, hq, hkv, d = 6, 9, 4, 2, 8
    ctx = history + rows
    group = hq // hkv
    # q = 0: uniform weights, out[i] = mean of V over keys 0 .. H + i
    q = np.zeros((rows, hq, d))
    k = rng.standard_normal((ctx, hkv, d))
    v = rng.standard_normal((ctx, hkv, d))
    got = orc.causal_attention(q, k, v, history)
    for i in range(rows):
        for h in range(hq):
            ref = v[:history + i + 1, h // group].mean(axis=0)
            assert np.max(np.abs(got[i, h] - ref)) <= 1e-14
    # every key equal: uniform weights again, whatever q is
    q = rng.standard_normal((rows, hq, d))
    k_same = np.broadcast_to(rng.standard_normal((1, hkv, d)), (ctx, hkv, d)).copy()
    got = orc.causal_attention(q, k_same, v, history)
    for i in range(rows):
        for h in range(hq):
            ref = v[:history + i + 1, h // group].mean(axis=0)
            assert np.max(np.abs(got[i, h] - ref)) <= 1e-14
    # constant V: the output is that constant
    const = rng.standard_normal((hkv, d))
    v_const = np.broadcast_to(const[None], (ctx, hkv, d)).copy()
    got = orc.causal_attention(q, k, v_const, history)
    for h in range(hq):
        assert np.max(np.abs(got[:, h] - const[h // group][None])) <= 1e-14
    # no history: the first row sees only key 0
    got = orc.causal_attention(q, k, v, 0)
    for h in range(hq):
        assert np.max(np.abs(got[0, h] - v[0, h // group])) <= 1e-15
    # one key with a score margin of about 60 dominates every row
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q_same = np.broadcast_to(u * math.sqrt(d), (rows, hq, d)).copy()
    k_small = rng.standard_normal((ctx, hkv, d)) * 0.01
    star = 3
    k_small[star] = u * 60.0
    got = orc.causal_attention(q_same, k_small, v, history)
    for i in range(rows):
        for h in range(hq):
            assert np.max(np.abs(got[i, h] - v[star, h // group])) <= 1e-15


def pin_weights(orc):
    """V = identity rows recovers the softmax weights: each row sums to 1,
    keys past H + i get exactly 0, and the weights match brute force."""
    rng = np.random.default_rng(14)
    rows, history, hq, hkv = 5, 7, 2, 1
    ctx = history + rows
    d = ctx + 3
    q = rng.standard_normal((rows, hq, d))
    k = rng.standard_normal((ctx, hkv, d))
    v = np.zeros((ctx, hkv, d))
    for j in range(ctx):
        v[j, 0, j] = 1.0
    p = orc.causal_attention(q, k, v, history)
    for i in range(rows):
        for h in range(hq):
            w = p[i, h]
            assert abs(w.sum() - 1.0) <= 1e-12
            assert np.all(w >= 0.0)
            assert np.all(w[history + i + 1:] == 0.0)
            s = [float(q[i, h] @ k[j, 0]) / math.sqrt(d) for j in range(history + i + 1)]
            e = [math.exp(x) for x in s]
            z = math.fsum(e)
            assert np.max(np.abs(w[:history + i + 1] - np.array(e) / z)) <= 1e-14


def pin_torch_sdpa(orc):
    """torch's CPU scaled_dot_product_attention in float64 with an explicit
    bottom-right causal mask (not is_causal, which aligns top-left when the
    query and key lengths differ) and KV heads repeated for GQA."""
    import torch
    rng = np.random.default_rng(15)
    for rows, history, hq, hkv, d in [(37, 100, 8, 2, 32), (16, 0, 4, 4, 16), (9, 61, 6, 2, 24)]:
        ctx = history + rows
        q = rng.standard_normal((rows, hq, d))
        k = rng.standard_normal((ctx, hkv, d))
        v = rng.standard_normal((ctx, hkv, d))
        tq = torch.from_numpy(q).permute(1, 0, 2)
        tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        mask = torch.arange(ctx)[None, :] <= (history + torch.arange(rows))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
        ref = ref.permute(1, 0, 2).numpy()
        got = orc.causal_attention(q, k, v, history)
        assert np.max(np.abs(got - ref)) <= 1e-12, np.max(np.abs(got - ref))


def pin_layout_invariance(orc):
    """Identity, permuted and pool-scattered block tables and contiguous KV
    give bitwise-identical outputs (the gather is exact)."""
    rng = np.random.default_rng(16)
    rows, history, hq, hkv, d, ps = 11, 45, 4, 2, 8, 4
    q, k, v, kp, vp, bt = paged_inputs(rng, rows, history, hq, hkv, d, ps, extra_pool=20)
    ctx = history + rows
    n_pages = -(-ctx // ps)
    ident = np.arange(n_pages, dtype=np.int32)
    kpi = np.full((n_pages, ps, hkv, d), np.nan)
    vpi = np.full((n_pages, ps, hkv, d), np.nan)
    for j in range(ctx):
        kpi[j // ps, j % ps] = k[j]
        vpi[j // ps, j % ps] = v[j]
    a = orc.paged_causal_attention(q, kp, vp, bt, history, ps)
    b = orc.paged_causal_attention(q, kpi, vpi, ident, history, ps)
    c = orc.causal_attention(q, k, v, history)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def pin_split_invariance(orc):
    """The split form with any number of page-aligned ranges, empty ones
    included, equals the direct form."""
    rng = np.random.default_rng(17)
    for rows, history, hq, hkv, d, ps in [(12, 50, 4, 1, 8, 4), (5, 0, 2, 2, 4, 2), (9, 33, 6, 2, 8, 8)]:
        ctx = history + rows
        q = rng.standard_normal((rows, hq, d))
        k = rng.standard_normal((ctx, hkv, d))
        v = rng.standard_normal((ctx, hkv, d))
        ref = orc.causal_attention(q, k, v, history)
        for n_splits in (1, 2, 3, 4, 7, 16, 32):
            ranges = orc.page_aligned_split_ranges(ctx, ps, n_splits)
            covered = sorted((a, b) for a, b in ranges if b > a)
            assert covered[0][0] == 0 and covered[-1][1] == ctx
            assert all(covered[t][1] == covered[t + 1][0] for t in range(len(covered) - 1))
            assert all(a % ps == 0 for a, b in ranges if b > a)
            got = orc.split_causal_attention(q, k, v, history, ranges)
            assert max_rel(got, ref) <= 1e-13, (n_splits, max_rel(got, ref))


def pin_split_partials(orc):
    """A range no row can see yields lse = -inf and O = 0; one full range
    yields lse = log of the softmax denominator (brute force)."""
    rng = np.random.default_rng(18)
    rows, history, hq, hkv, d = 4, 6, 2, 1, 4
    ctx = history + rows
    q = rng.standard_normal((rows, hq, d))
    k = rng.standard_normal((ctx, hkv, d))
    v = rng.standard_normal((ctx, hkv, d))
    # keys [history + 1, ctx) are invisible to row 0
    o_part, lse = orc.split_partials(q, k, v, history, [(0, history + 1), (history + 1, ctx)])
    assert np.all(lse[1, 0] == -np.inf) and np.all(o_part[1, 0] == 0.0)
    for i in range(1, rows):
        assert np.all(np.isfinite(lse[1, i]))
    o_full, lse_full = orc.split_partials(q, k, v, history, [(0, ctx)])
    for i in range(rows):
        for h in range(hq):
            s = [float(q[i, h] @ k[j, 0]) / math.sqrt(d) for j in range(history + i + 1)]
            assert abs(lse_full[0, i, h] - math.log(math.fsum(math.exp(x) for x in s))) <= 1e-13


def pin_piece_invariance(orc):
    """Cutting the chunk into pieces (call i: rows [iP, (i+1)P) at history
    H + iP over the same K/V) equals one call."""
    rng = np.random.default_rng(19)
    rows, history, hq, hkv, d = 32, 21, 4, 2, 8
    ctx = history + rows
    q = rng.standard_normal((rows, hq, d))
    k = rng.standard_normal((ctx, hkv, d))
    v = rng.standard_normal((ctx, hkv, d))
    ref = orc.causal_attention(q, k, v, history)
    for piece in (1, 5, 8, 16):
        parts = [orc.causal_attention(q[s:s + piece], k, v, history + s) for s in range(0, rows, piece)]
        assert max_rel(np.concatenate(parts), ref) <= 1e-13


def pin_causality(orc):
    """Changing K/V after position H + i leaves row i bit-for-bit unchanged and
    changes later rows."""
    rng = np.random.default_rng(20)
    rows, history, hq, hkv, d = 8, 10, 2, 1, 4
    ctx = history + rows
    q = rng.standard_normal((rows, hq, d))
    k = rng.standard_normal((ctx, hkv, d))
    v = rng.standard_normal((ctx, hkv, d))
    base = orc.causal_attention(q, k, v, history)
    i = 3
    k2, v2 = k.copy(), v.copy()
    k2[history + i + 1:] += 5.0
    v2[history + i + 1:] -= 3.0
    pert = orc.causal_attention(q, k2, v2, history)
    assert np.array_equal(pert[:i + 1], base[:i + 1])
    assert np.all(np.abs(pert[i + 1:] - base[i + 1:]).max(axis=(1, 2)) > 1e-6)


def pin_gqa_is_mha_with_repeated_kv(orc):
    rng = np.random.default_rng(21)
    rows, history, hq, hkv, d = 6, 14, 6, 2, 8
    ctx = history + rows
    q = rng.standard_normal((rows, hq, d))
    k = rng.standard_normal((ctx, hkv, d))
    v = rng.standard_normal((ctx, hkv, d))
    gqa = orc.causal_attention(q, k, v, history)
    mha = orc.causal_attention(q, np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1), history)
    assert max_rel(gqa, mha) <= 1e-13
    # and the head map is h -> h div G: swapping the two KV heads swaps the outputs of the groups
    swapped = orc.causal_attention(q[:, ::-1].copy(), k[:, ::-1].copy(), v[:, ::-1].copy(), history)
    assert max_rel(swapped[:, ::-1], gqa) <= 1e-13


def pin_row_subset(orc):
    rng = np.random.default_rng(22)
    rows, history, hq, hkv, d = 40, 30, 4, 1, 8
    ctx = history + rows
    q = rng.standard_normal((rows, hq, d))
    k = rng.standard_normal((ctx, hkv, d))
    v = rng.standard_normal((ctx, hkv, d))
    full = orc.causal_attention(q, k, v, history)
    sel = np.array([39, 0, 17, 5])
    got = orc.causal_attention_rows(q, k, v, history, sel)
    assert max_rel(got, full[sel]) <= 1e-13


def load_golden(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append([int(x) for x in line.split()])
    return out


def pin_page_split_table(rules):
    for cores, kv_heads, piece_rows, tiles, splits in load_golden("page_split_table.txt"):
        assert tiles == piece_rows // 8
        assert rules.page_split_rule(cores, kv_heads, tiles) == splits, (cores, kv_heads, piece_rows)


def pin_page_piece_rows(rules):
    for history, piece in load_golden("page_piece_rows.txt"):
        assert rules.page_piece_rows(history) == piece, history


# ---------------------------------------------------------------- KV append
def _append_case(rng, history, rows, hkv, d, ps, extra_pool=3):
    """A pool holding H tokens through a permuted table, every other slot
    poisoned with NaN, and R new rows to append."""
    ctx = history + rows
    n_pages = max(1, -(-ctx // ps))
    pool = n_pages + extra_pool
    bt = rng.permutation(pool)[:n_pages].astype(np.int32)
    kp = np.full((pool, ps, hkv, d), np.nan)
    vp = np.full((pool, ps, hkv, d), np.nan)
    k_hist = rng.standard_normal((history, hkv, d))
    v_hist = rng.standard_normal((history, hkv, d))
    for j in range(history):
        kp[bt[j // ps], j % ps] = k_hist[j]
        vp[bt[j // ps], j % ps] = v_hist[j]
    k_new = rng.standard_normal((rows, hkv, d))
    v_new = rng.standard_normal((rows, hkv, d))
    return kp, vp, bt, k_hist, v_hist, k_new, v_new


APPEND_SHAPES = [
    # history, rows, Hkv, d, ps: page-aligned and not, one-token pages, a chunk inside one page
    (0, 5, 1, 4, 2), (3, 6, 2, 3, 4), (8, 8, 1, 2, 4), (5, 1, 3, 2, 1), (2, 3, 2, 4, 16), (17, 30, 2, 5, 8),
]


def pin_append_gather(orc):
    """After the append, reading the cache back through the block table (the
    gather, pinned above) gives the old history followed by the new rows, and
    every pool slot outside positions 0 .. H+R-1 keeps its old bits."""
    import oracle as real
    rng = np.random.default_rng(21)
    for history, rows, hkv, d, ps in APPEND_SHAPES:
        kp, vp, bt, k_hist, v_hist, k_new, v_new = _append_case(rng, history, rows, hkv, d, ps)
        k_out, v_out = orc.kv_append(kp, vp, bt, history, ps, k_new, v_new)
        ctx = history + rows
        assert np.array_equal(real.gather_pages(k_out, bt, ctx, ps), np.concatenate([k_hist, k_new]))
        assert np.array_equal(real.gather_pages(v_out, bt, ctx, ps), np.concatenate([v_hist, v_new]))
        touched = np.zeros(kp.shape[:2], dtype=bool)
        for j in range(ctx):
            touched[bt[j // ps], j % ps] = True
        assert np.array_equal(k_out[~touched], kp[~touched], equal_nan=True)
        assert np.array_equal(v_out[~touched], vp[~touched], equal_nan=True)
        # the inputs are not modified: the new rows' slots still hold NaN there
        for i in range(rows):
            pos = history + i
            assert np.isnan(kp[bt[pos // ps], pos % ps]).all() and np.isnan(vp[bt[pos // ps], pos % ps]).all()


def pin_append_pieces(orc):
    """Appending R1 rows and then R2 rows at H + R1 equals appending R1 + R2
    rows at once; appending nothing changes nothing."""
    rng = np.random.default_rng(22)
    kp, vp, bt, _, _, k_new, v_new = _append_case(rng, 7, 12, 2, 3, 4)
    k1, v1 = orc.kv_append(kp, vp, bt, 7, 4, k_new, v_new)
    k2, v2 = orc.kv_append(kp, vp, bt, 7, 4, k_new[:5], v_new[:5])
    k2, v2 = orc.kv_append(k2, v2, bt, 12, 4, k_new[5:], v_new[5:])
    assert np.array_equal(k1, k2, equal_nan=True) and np.array_equal(v1, v2, equal_nan=True)
    k0, v0 = orc.kv_append(kp, vp, bt, 7, 4, k_new[:0], v_new[:0])
    assert np.array_equal(k0, kp, equal_nan=True) and np.array_equal(v0, vp, equal_nan=True)


def pin_append_contiguous(orc):
    """With an identity table the pool is the contiguous layout: rows H ..
    H+R-1 of its [tokens][Hkv][d] view are the new rows, bit for bit (16-bit
    patterns, NaN payloads and -0 included)."""
    rng = np.random.default_rng(23)
    ps, hkv, d, history, rows = 4, 2, 3, 6, 9
    n_pages = -(-(history + rows) // ps)
    kp = rng.integers(0, 1 << 16, size=(n_pages, ps, hkv, d), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(n_pages, ps, hkv, d), dtype=np.uint16)
    k_new = rng.integers(0, 1 << 16, size=(rows, hkv, d), dtype=np.uint16)
    k_new[0, 0, :] = [0x7E01, 0x8000, 0xFC00]
    v_new = rng.integers(0, 1 << 16, size=(rows, hkv, d), dtype=np.uint16)
    bt = np.arange(n_pages, dtype=np.int32)
    k_out, v_out = orc.kv_append(kp, vp, bt, history, ps, k_new, v_new)
    kc, vc = k_out.reshape(-1, hkv, d), v_out.reshape(-1, hkv, d)
    assert np.array_equal(kc[history:history + rows], k_new) and np.array_equal(vc[history:history + rows], v_new)
    assert np.array_equal(kc[:history], kp.reshape(-1, hkv, d)[:history])
    assert np.array_equal(vc[history + rows:], vp.reshape(-1, hkv, d)[history + rows:])


CACHE_PINS = [pin_append_gather, pin_append_pieces, pin_append_contiguous]


# ---------------------------------------------------------------- varlen
UNUSED_ENTRY = 1 << 30   # block-table padding: indexing the pool with it raises


def varlen_batch(rng, seqs, hq, hkv, d, ps, extra_pool=4):
    """A packed batch of sequences [(history, rows)] over one NaN-poisoned
    pool: each sequence gets its own pages in random pool order, its table row
    padded with an entry that cannot be read.  Returns q, k_pages, v_pages,
    block_tables, cu_rows, histories and the per-sequence contiguous (k, v)."""
    n_pages = [max(1, -(-(h + r) // ps)) for h, r in seqs]
    pool = sum(n_pages) + extra_pool
    order = rng.permutation(pool)
    width = max(n_pages)
    tables = np.full((len(seqs), width), UNUSED_ENTRY, dtype=np.int64)
    k_pages = np.full((pool, ps, hkv, d), np.nan)
    v_pages = np.full((pool, ps, hkv, d), np.nan)
    kv = []
    at = 0
    for s, (h, r) in enumerate(seqs):
        tables[s, :n_pages[s]] = order[at:at + n_pages[s]]
        at += n_pages[s]
        k = rng.standard_normal((h + r, hkv, d))
        v = rng.standard_normal((h + r, hkv, d))
        for j in range(h + r):
            k_pages[tables[s, j // ps], j % ps] = k[j]
            v_pages[tables[s, j // ps], j % ps] = v[j]
        kv.append((k, v))
    cu = np.concatenate([[0], np.cumsum([r for _, r in seqs])]).astype(np.int64)
    q = rng.standard_normal((int(cu[-1]), hq, d))
    hist = np.array([h for h, _ in seqs], dtype=np.int64)
    return q, k_pages, v_pages, tables, cu, hist, kv


VARLEN_SEQS = [(5, 3), (0, 4), (13, 0), (2, 1), (9, 2)]


def pin_varlen_brute_force(orc):
    """Each sequence's rows equal the brute-force definition over that
    sequence's own table and history (a batch with an empty sequence, a first
    chunk, non-aligned histories)."""
    rng = np.random.default_rng(31)
    for hq, hkv, d, ps in ((4, 2, 3, 2), (3, 1, 4, 4)):
        q, kp, vp, bt, cu, hist, _ = varlen_batch(rng, VARLEN_SEQS, hq, hkv, d, ps)
        got = orc.varlen_paged_attention(q, kp, vp, bt, cu, hist, ps)
        assert got.shape == q.shape
        for s, (h, r) in enumerate(VARLEN_SEQS):
            if r == 0:
                continue
            want = brute_force(q[cu[s]:cu[s + 1]], kp, vp, bt[s], h, ps)
            assert max_rel(got[cu[s]:cu[s + 1]], want) < 1e-12, (s, h, r)


def pin_varlen_sharing_and_isolation(orc):
    """Two sequences naming the same pool pages with the same rows get the
    same output (a shared prefix is read by both); poisoning the pages of a
    third sequence leaves the first two bit-identical and makes only the
    third's rows NaN."""
    rng = np.random.default_rng(32)
    ps = 2
    q, kp, vp, bt, cu, hist, _ = varlen_batch(rng, [(6, 3), (6, 3), (4, 2)], 4, 2, 3, ps)
    bt[1] = bt[0]
    q[cu[1]:cu[2]] = q[cu[0]:cu[1]]
    base = orc.varlen_paged_attention(q, kp, vp, bt, cu, hist, ps)
    assert np.array_equal(base[cu[0]:cu[1]], base[cu[1]:cu[2]])
    assert np.all(np.isfinite(base))
    n2 = -(-(hist[2] + cu[3] - cu[2]) // ps)
    kp2 = kp.copy()
    kp2[bt[2, :n2]] = np.nan
    got = orc.varlen_paged_attention(q, kp2, vp, bt, cu, hist, ps)
    assert np.array_equal(got[:cu[2]], base[:cu[2]])
    assert np.all(np.isnan(got[cu[2]:cu[3]]))


def pin_varlen_permutation(orc):
    """Reordering the sequences of a batch (rows, tables, histories together)
    reorders the output's row blocks the same way, bit for bit."""
    rng = np.random.default_rng(33)
    ps = 4
    q, kp, vp, bt, cu, hist, _ = varlen_batch(rng, VARLEN_SEQS, 4, 2, 3, ps)
    base = orc.varlen_paged_attention(q, kp, vp, bt, cu, hist, ps)
    perm = [3, 0, 4, 2, 1]
    rows = [np.arange(cu[s], cu[s + 1]) for s in perm]
    q2 = q[np.concatenate(rows)]
    cu2 = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    got = orc.varlen_paged_attention(q2, kp, vp, bt[perm], cu2, hist[perm], ps)
    assert np.array_equal(got, base[np.concatenate(rows)])


VARLEN_PINS = [pin_varlen_brute_force, pin_varlen_sharing_and_isolation, pin_varlen_permutation]

ATTENTION_PINS = [
    pin_decoders, pin_gather, pin_brute_force, pin_closed_forms, pin_weights, pin_torch_sdpa,
    pin_layout_invariance, pin_split_invariance, pin_split_partials, pin_piece_invariance,
    pin_causality, pin_gqa_is_mha_with_repeated_kv, pin_row_subset,
]
RULE_PINS = [pin_page_split_table, pin_page_piece_rows]


# ---------------------------------------------------------------- q8 pages
def load_q8_golden():
    vals, qs, bits = [], [], None
    with open(os.path.join(GOLDEN, "q8_block.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            a, b = line.split()
            if a == "scale_bits":
                bits = int(b, 16)
            else:
                vals.append(float(a))
                qs.append(int(b))
    return vals, qs, bits


def pin_q8_golden_block(orc):
    """The hand-quantized block (tests/golden/q8_block.txt), as block 1 of a
    64-value row whose block 0 is all zero (scale 0, quants 0)."""
    vals, qs, bits = load_q8_golden()
    row = np.zeros(64)
    row[32:32 + len(vals)] = vals
    q, scale = orc.quantize_q8(row[None])
    assert q.dtype == np.int8 and q.shape == (1, 64) and scale.shape == (1, 2)
    want = np.zeros(64, dtype=np.int8)
    want[32:32 + len(qs)] = qs
    assert np.array_equal(q[0], want), q[0]
    assert np.asarray(scale, dtype=np.float16).view(np.uint16)[0, 1] == bits
    assert float(scale[0, 0]) == 0.0


def pin_q8_round_trip(orc):
    """For random blocks over six orders of magnitude (fp16-exact values):
    every value comes back within half a step (|scale q - x| <= scale / 2),
    the block's largest |x| maps to +-127, and (scales in fp16's normal
    range) scaling a block by 4 scales its scale by 4 and leaves its quants
    unchanged."""
    rng = np.random.default_rng(41)
    for mag in (1e-3, 0.1, 1.0, 30.0, 500.0):
        x = (rng.standard_normal((7, 3, 128)) * mag).astype(np.float16).astype(np.float64)
        q, scale = orc.quantize_q8(x)
        back = orc.dequantize_q8(q, scale)
        step = np.repeat(np.asarray(scale, dtype=np.float64), 32, axis=-1)
        assert np.all(np.abs(back - x) <= step / 2 + 1e-300), mag
        qb = np.abs(q.astype(np.int64)).reshape(7, 3, 4, 32).max(axis=-1)
        assert np.all(qb == 127), mag
        if mag >= 0.1:   # scales in fp16's normal range (subnormals round on a fixed grid)
            q2, scale2 = orc.quantize_q8(x * 4.0)
            assert np.array_equal(q2, q)
            assert np.array_equal(np.asarray(scale2, np.float64), 4.0 * np.asarray(scale, np.float64))


def pin_q8_exact_multiples_and_saturation(orc):
    """Blocks of integer multiples k s of an fp16 step s (max |k| = 127) come
    back exactly, with scale s; all-zero blocks give scale 0 and quants 0;
    beyond fp16 range the scale saturates at 65504 and quants at +-127."""
    rng = np.random.default_rng(42)
    for s in (2.0 ** -9, 0.375, 3.0):
        k = rng.integers(-127, 128, size=(5, 64))
        k[:, 0] = 127
        k[:, 40] = -127
        q, scale = orc.quantize_q8(k * s)
        assert np.array_equal(q.astype(np.int64), k) and np.all(np.asarray(scale, np.float64) == s)
    q, scale = orc.quantize_q8(np.zeros((2, 64)))
    assert not q.any() and not np.asarray(scale, np.float64).any()
    big = np.zeros((1, 32))
    big[0, :3] = [1.0e7, -2.0e7, 1.0e3]
    q, scale = orc.quantize_q8(big)
    assert float(scale[0, 0]) == 65504.0
    assert list(q[0, :3]) == [127, -127, 0]


def _binary16_value(bits):
    """The value of an IEEE 754 binary16 bit pattern from its fields: sign
    bit 15, biased exponent bits 14..10 (bias 15), fraction bits 9..0;
    exponent 0 is a subnormal (fraction * 2^-24), exponent 31 is infinity
    (fraction 0) or NaN."""
    sign = -1.0 if bits >> 15 else 1.0
    exp = (bits >> 10) & 0x1F
    frac = bits & 0x3FF
    if exp == 0x1F:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(frac, -24)
    return sign * math.ldexp(1024 + frac, exp - 25)


def pin_q8_decode_scales(orc):
    """Scale bit patterns decode to the binary16 values their fields define:
    known patterns (the golden block's 0x2008 = 129/16384, 1, the largest
    finite 65504, the smallest subnormal, signed zero, infinity, NaN) and
    random patterns over the whole 16-bit range, each against the value
    computed from its sign, exponent and fraction fields."""
    known = {0x2008: 129 / 16384, 0x3C00: 1.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24, 0x0400: 2.0 ** -14,
             0x8000: -0.0, 0xC000: -2.0, 0x7C00: math.inf, 0xFC00: -math.inf}
    raw = np.array(list(known), dtype=np.uint16)
    got = np.asarray(orc.decode_scales(raw)).astype(np.float64)
    want = np.array(list(known.values()))
    assert np.array_equal(got, want), got
    assert np.array_equal(np.signbit(got), np.signbit(want))
    for nan_bits in (0xFFFF, 0x7E00, 0x7C01):
        assert math.isnan(float(np.asarray(orc.decode_scales(np.array([nan_bits], dtype=np.uint16)))[0]))
    rng = np.random.default_rng(45)
    raw = rng.integers(0, 1 << 16, size=2048).astype(np.uint16)
    got = np.asarray(orc.decode_scales(raw)).astype(np.float64)
    want = np.array([_binary16_value(int(b)) for b in raw])
    finite = ~np.isnan(want)
    assert np.array_equal(np.isnan(got), ~finite)
    assert np.array_equal(got[finite], want[finite])


def _q8_pool(rng, history, rows, hkv, d, ps, extra_pool=2):
    ctx = history + rows
    n_pages = -(-ctx // ps)
    pool = n_pages + extra_pool
    bt = rng.permutation(pool)[:n_pages].astype(np.int32)
    kq = rng.integers(-127, 128, size=(pool, ps, hkv, d)).astype(np.int8)
    vq = rng.integers(-127, 128, size=(pool, ps, hkv, d)).astype(np.int8)
    ks = (rng.random((pool, ps, hkv, d // 32)) * 0.02 + 0.001).astype(np.float16)
    vs = (rng.random((pool, ps, hkv, d // 32)) * 0.02 + 0.001).astype(np.float16)
    return kq, ks, vq, vs, bt


def pin_q8_attention(orc):
    """Attention over q8 pages equals brute force over the dequantized pages
    (tiny shapes), and equals the 16-bit attention of the dequantized
    contiguous K/V with the table permuted."""
    import oracle as real
    rng = np.random.default_rng(43)
    for rows, history, hq, hkv, d, ps in ((4, 9, 4, 2, 32, 4), (3, 0, 2, 1, 64, 2), (5, 20, 6, 3, 32, 8)):
        kq, ks, vq, vs, bt = _q8_pool(rng, history, rows, hkv, d, ps)
        q = rng.standard_normal((rows, hq, d))
        got = orc.paged_q8_attention(q, kq, ks, vq, vs, bt, history, ps)
        kd = orc.dequantize_q8(kq, ks)
        vd = orc.dequantize_q8(vq, vs)
        assert max_rel(got, brute_force(q, kd, vd, bt, history, ps)) < 1e-12
        ctx = history + rows
        kc = real.dequantize_q8(real.gather_pages(kq, bt, ctx, ps), real.gather_pages(ks, bt, ctx, ps))
        vc = real.dequantize_q8(real.gather_pages(vq, bt, ctx, ps), real.gather_pages(vs, bt, ctx, ps))
        assert max_rel(got, real.causal_attention(q, kc, vc, history)) < 1e-12


def pin_q8_append(orc):
    """Quantizing appends: the new rows' quants and scales read back through
    the table are quantize_q8 of the rows; other slots keep their bits; two
    appends in a row equal one."""
    import oracle as real
    rng = np.random.default_rng(44)
    for history, rows, hkv, d, ps in ((5, 7, 2, 64, 4), (0, 3, 1, 32, 2), (16, 16, 2, 32, 16)):
        kq, ks, vq, vs, bt = _q8_pool(rng, history, rows, hkv, d, ps)
        ks, vs = ks.view(np.uint16), vs.view(np.uint16)
        kn = rng.standard_normal((rows, hkv, d)).astype(np.float16).astype(np.float64)
        vn = rng.standard_normal((rows, hkv, d)).astype(np.float16).astype(np.float64)
        out = orc.kv_append_q8(kq, ks, vq, vs, bt, history, ps, kn, vn)
        wq, wsc = real.quantize_q8(kn)
        ctx = history + rows
        assert np.array_equal(real.gather_pages(out[0], bt, ctx, ps)[history:], wq)
        assert np.array_equal(real.gather_pages(out[1], bt, ctx, ps)[history:], wsc.view(np.uint16))
        wq, wsc = real.quantize_q8(vn)
        assert np.array_equal(real.gather_pages(out[2], bt, ctx, ps)[history:], wq)
        assert np.array_equal(real.gather_pages(out[3], bt, ctx, ps)[history:], wsc.view(np.uint16))
        touched = np.zeros(kq.shape[:2], dtype=bool)
        for j in range(history, ctx):
            touched[bt[j // ps], j % ps] = True
        for a, b in zip(out, (kq, ks, vq, vs)):
            assert np.array_equal(a[~touched], b[~touched])
        half = rows // 2
        two = orc.kv_append_q8(kq, ks, vq, vs, bt, history, ps, kn[:half], vn[:half])
        two = orc.kv_append_q8(*two, bt, history + half, ps, kn[half:], vn[half:])
        assert all(np.array_equal(a, b) for a, b in zip(out, two))


QUANT_PINS = [pin_q8_golden_block, pin_q8_decode_scales, pin_q8_round_trip, pin_q8_exact_multiples_and_saturation, pin_q8_attention,
              pin_q8_append]
