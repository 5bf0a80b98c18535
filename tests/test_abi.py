"""CPU-side checks of the C ABI: the library loads, exports every function
include/paged_prefill.h declares, and its host-only helpers (planner, split
rule, piece rule, block-table check, argument checks) behave as documented.
No call here reaches a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import _pins
import paged_kv_prefill_amd as pkg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("paged_", "contiguous_"))))


def test_library_exports_every_declared_symbol():
    lib = pkg.lib()
    names = declared_functions()
    assert len(names) == 19, names
    for name in names:
        assert hasattr(lib, name), name
    assert lib.paged_prefill_version() == 10100


def test_binding_covers_every_declared_symbol():
    for name in declared_functions():
        assert name in pkg._SIGNATURES, name


def _merge_pairs_per_block(d, n_splits):
    """The merge kernel serves a (row, head) pair with groups of d/4 threads:
    16 groups from 64 splits, 4 from 16, else 1; a block has max(256, threads
    per pair) threads."""
    groups = 16 if n_splits >= 64 else 4 if n_splits >= 16 else 1
    per_pair = d // 4 * groups
    return max(256, per_pair) // per_pair


def test_split_rule_reproduces_the_pr_table():
    for cores, kv_heads, piece_rows, tiles, splits in _pins.load_golden("page_split_table.txt"):
        assert pkg.paged_prefill_split_rule(cores, kv_heads, tiles) == splits


def test_piece_rows_reproduce_the_pr_sizes():
    for history, piece in _pins.load_golden("page_piece_rows.txt"):
        assert pkg.paged_prefill_piece_rows(history) == piece


def test_plan_matches_the_workloads():
    # 2048-row chunk, 16/2 heads, d 256: 128 m-tiles x 2 KV heads fill 256 CUs with one split
    p = pkg.paged_prefill_plan(32768, 2048, 16, 2, 256)
    assert p["n_splits"] == 1 and p["grid"] == 256 and p["workspace_bytes"] == 0
    # 256-row piece, 32/4 heads, d 128: 256-vector m tiles (two query blocks per
    # wave), 8 m-tiles x 4 heads -> 8 splits
    p = pkg.paged_prefill_plan(65536, 256, 32, 4, 128)
    assert p["m_tile"] == 256 and p["n_splits"] == 8 and p["grid"] == 256
    # 128-row piece, 16/2 heads, d 256 at 128K: 8 x 2 -> 16 splits, the PR's count at 128K
    p = pkg.paged_prefill_plan(131072, 128, 16, 2, 256)
    assert p["n_splits"] == 16 and p["grid"] == 256
    assert p["workspace_bytes"] <= 2048 * 16 * 257 * 4 + 512


def _check_plan(history, rows, hq, hkv, d, ps, req, p):
    """The documented shape of a single-call plan."""
    ctx = history + rows
    g = hq // hkv
    # calls with at most 16 query vectors per KV head and pages of >= 8 tokens
    # get the narrow kernel: 32-key tiles, one 32-vector m tile, one workgroup
    # per (split, KV head)
    narrow = rows * g <= 16 and ps >= 8
    assert (p["m_tile"] == 32) == narrow, p
    tile = 32 if narrow else 64
    unit = max(tile, ps)
    assert p["split_tokens"] % tile == 0 and p["split_tokens"] % ps == 0
    assert p["kv_tile"] == tile
    # the splits cover [0, ctx) and none is empty
    assert (p["n_splits"] - 1) * p["split_tokens"] < ctx <= p["n_splits"] * p["split_tokens"]
    if req:
        # clamped to the key axis's units; the narrow kernel's splits hold at
        # most 128 pages, which may raise a small request
        floor = -(-ctx // (128 * ps)) if narrow else 1
        assert p["n_splits"] <= max(1, min(req, -(-ctx // unit)), floor)
    if narrow:
        assert 1 <= p["n_splits"] <= 4096
        assert p["m_tile"] == 32 and p["tiles_m"] == 1
        assert p["split_tokens"] // ps <= 128          # the pages a split keeps in registers
        if not req and p["split_tokens"] < 128 * ps:   # not bound by the page registers
            assert p["grid"] <= 256 + hkv
            assert p["n_splits"] <= max(1, -(-ctx // 256))   # at most one split per 256 keys
    else:
        # two query blocks per wave (256-vector m tiles) at d <= 128 once the
        # call has more query vectors than one 128-vector tile
        assert p["m_tile"] == (256 if d <= 128 and rows * g > 128 else 128)
        assert p["tiles_m"] == -(-rows * g // p["m_tile"])
        if not req:
            # one workgroup per CU over the KV heads and m tiles, at most 128
            # splits, and never more partials than a full 2048-row chunk's
            assert p["n_splits"] <= max(1, min(128, (256 // hkv) // p["tiles_m"]))
            assert p["workspace_bytes"] <= 2 * 2048 * hq * (d + 1) * 4 + 1024
    assert p["grid"] == p["tiles_m"] * hkv * p["n_splits"]
    if p["n_splits"] > 1:
        assert p["workspace_bytes"] >= p["n_splits"] * rows * hq * (d + 1) * 4
        assert p["merge_grid"] == -(-rows * hq // _merge_pairs_per_block(d, p["n_splits"]))
    else:
        assert p["workspace_bytes"] == 0 and p["merge_grid"] == 0


@pytest.mark.parametrize("history,rows,hq,hkv,d,ps,req", [
    (0, 1, 1, 1, 64, 16, 0), (5, 3, 4, 1, 64, 1, 0), (512, 64, 4, 1, 64, 16, 4), (1000, 77, 6, 2, 128, 8, 0),
    (131072, 128, 16, 2, 256, 16, 0), (100, 2048, 32, 4, 128, 256, 0), (37, 5, 16, 2, 256, 16, 64),
    (8192, 512, 16, 2, 256, 16, 0), (65536, 2048, 32, 8, 128, 16, 0), (3, 1, 2, 2, 64, 1024, 5),
    (4000, 3, 16, 2, 128, 16, 0), (4000, 2, 8, 1, 256, 32, 0),   # 24 and 16 query vectors per KV head
])
def test_plan_invariants(history, rows, hq, hkv, d, ps, req):
    _check_plan(history, rows, hq, hkv, d, ps, req, pkg.paged_prefill_plan(history, rows, hq, hkv, d, ps, req))


PS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]


@settings(max_examples=400, deadline=None, derandomize=True, database=None)
@given(history=st.integers(0, 1 << 20), rows=st.integers(1, 4096), hkv=st.sampled_from([1, 2, 4, 8]),
       g=st.sampled_from([1, 2, 4, 8]), d=st.sampled_from([64, 128, 256]), ps=st.sampled_from(PS),
       req=st.one_of(st.just(0), st.integers(1, 256)))
def test_plan_invariants_random(history, rows, hkv, g, d, ps, req):
    """The same over random shapes (histories up to 1M, where no decode plan
    passes the split or workspace limits).  A requested split count may ask
    for more workspace than the cap: then the call is refused."""
    hq = hkv * g
    try:
        p = pkg.paged_prefill_plan(history, rows, hq, hkv, d, ps, req)
    except pkg.PagedPrefillError as e:
        # only a requested count is refused: its partials would pass the
        # workspace cap (-5) or the 32-bit element index of the workspace (-10)
        assert e.code in (-5, -10) and req > 0, e
        n_units = -(-(history + rows) // max(32 if rows * g <= 16 and ps >= 8 else 64, ps))
        partials = min(req, n_units) * rows * hq
        assert partials * (d + 1) * 4 > 2 ** 31 if e.code == -5 else partials * d >= 2 ** 31
        return
    _check_plan(history, rows, hq, hkv, d, ps, req, p)


@pytest.mark.parametrize("history,hq,hkv,d,ps", [
    (131072, 16, 2, 256, 16), (65536, 32, 4, 128, 16), (32768, 16, 2, 256, 16), (1 << 22, 8, 1, 64, 16),
    (100000, 8, 1, 128, 8), (5000, 64, 8, 128, 32), (300, 16, 2, 256, 64)])
def test_narrow_plans(history, hq, hkv, d, ps):
    """Decode steps and appends of up to 16 query vectors per KV head (16-bit
    K/V): about one workgroup per CU (256), no split under 256 keys unless the
    context is shorter, whole pages and at most 128 of them per split."""
    g = hq // hkv
    for rows in sorted({1, max(1, 16 // g)}):
        p = pkg.paged_prefill_plan(history, rows, hq, hkv, d, ps)
        ctx = history + rows
        assert p["m_tile"] == 32 and p["kv_tile"] == 32
        assert p["split_tokens"] % max(32, ps) == 0 and p["split_tokens"] // ps <= 128
        assert p["grid"] == hkv * p["n_splits"]
        if p["split_tokens"] < 128 * ps:   # not bound by the page registers
            assert p["grid"] <= 256 + hkv
            assert p["n_splits"] == 1 or p["split_tokens"] >= 256 - max(32, ps)
    # one vector past 16 per KV head: the prefill kernel
    p = pkg.paged_prefill_plan(history, 16 // g + 1, hq, hkv, d, ps)
    assert p["m_tile"] >= 128 and p["kv_tile"] == 64


def test_narrow_plan_past_the_workspace_cap_gives_way(monkeypatch):
    """A planner-chosen narrow plan whose split workspace would pass the cap
    (PPA_MAX_WORKSPACE_BYTES) gives way to the prefill kernel's plan, whose
    splits are capped by the full-chunk bound; a requested split count past
    the cap is an error."""
    args = (1 << 20, 1, 16, 2, 256, 16)   # one row at 1M history: 513 splits of 128 pages
    p = pkg.paged_prefill_plan(*args)
    assert p["m_tile"] == 32 and p["n_splits"] == 513
    monkeypatch.setenv("PPA_MAX_WORKSPACE_BYTES", str(p["workspace_bytes"] - 1))
    q = pkg.paged_prefill_plan(*args)
    assert q["m_tile"] >= 128 and 1 < q["n_splits"] < 513
    assert q["workspace_bytes"] < p["workspace_bytes"]
    with pytest.raises(pkg.PagedPrefillError) as e:
        pkg.paged_prefill_plan(*args, n_splits=513)
    assert e.value.code == -5   # PPA_ERR_WORKSPACE
    # a batch of 32 decode steps at up to 4M tokens, 64/8 heads, d 256: the
    # narrow plan (2048 splits of 128 pages over 32 rows) would need 4.3 GB,
    # past the default 2 GiB cap; the prefill plan's workspace is bounded
    monkeypatch.delenv("PPA_MAX_WORKSPACE_BYTES")
    v = pkg.paged_prefill_plan_varlen(32, 32, 1, 1 << 22, 64, 8, 256, 16)
    assert v["m_tile"] >= 128 and v["workspace_bytes"] <= 2 << 30


def test_planner_never_exceeds_a_full_chunk_workspace():
    for history in (1024, 8192, 32768, 65536, 131072, 262144):
        for rows in (1, 16, 128, 256, 512, 1024, 2048):
            for hq, hkv, d in ((16, 2, 256), (32, 4, 128), (4, 1, 64), (32, 8, 128)):
                p = pkg.paged_prefill_plan(history, rows, hq, hkv, d)
                assert p["n_splits"] * rows <= max(2048, rows) * 1 + 2048, (history, rows)
                assert p["workspace_bytes"] <= 2048 * hq * (d + 1) * 4 * 2 + 1024


def test_check_block_table():
    assert pkg.paged_prefill_check_block_table(np.array([0, 5, 3]), 6) == 0
    assert pkg.paged_prefill_check_block_table(np.array([0, 6, 3]), 6) == -7
    assert pkg.paged_prefill_check_block_table(np.array([-1]), 6) == -7
    assert pkg.paged_prefill_check_block_table(np.array([], dtype=np.int32), 6) == 0


def _call_paged(**kw):
    a = dict(q=16, kp=16, vp=16, bt=16, H=10, R=4, hq=4, hkv=2, d=64, ps=16, S=0, out=4096, dt=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return pkg.lib().paged_prefill_attention(vp(a["q"]), vp(a["kp"]), vp(a["vp"]), vp(a["bt"]), a["H"], a["R"],
                                             a["hq"], a["hkv"], a["d"], a["ps"], a["S"], vp(a["out"]), a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), -4), (dict(R=-1), -2), (dict(H=-5), -2), (dict(hq=5, hkv=2), -2), (dict(hkv=0), -2),
    (dict(d=96), -3), (dict(d=512), -3), (dict(ps=12), -3), (dict(ps=2048), -3), (dict(ps=0), -3),
    (dict(S=-1), -2), (dict(q=0), -1), (dict(bt=0), -1), (dict(out=0), -1), (dict(q=24), -8),
    (dict(out=16 + 64), -9), (dict(H=2 ** 31), -10),
])
def test_argument_errors_return_before_any_device_work(kw, code):
    assert _call_paged(**kw) == code
    assert pkg.strerror(code) not in ("unknown status", "ok")


def test_empty_chunk_is_a_no_op():
    assert _call_paged(R=0, q=0, kp=0, vp=0, bt=0, out=0) == 0


def _call_append(**kw):
    a = dict(kn=16, vn=32, kp=4096, vp=8192, bt=64, H=10, R=4, hkv=2, d=64, ps=16, dt=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return pkg.lib().paged_kv_append(vp(a["kn"]), vp(a["vn"]), vp(a["kp"]), vp(a["vp"]), vp(a["bt"]), a["H"],
                                     a["R"], a["hkv"], a["d"], a["ps"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), -4), (dict(R=-1), -2), (dict(H=-1), -2), (dict(hkv=0), -2), (dict(d=32), -3),
    (dict(ps=3), -3), (dict(ps=4096), -3), (dict(kn=0), -1), (dict(vp=0), -1), (dict(bt=0), -1),
    (dict(kn=24), -8), (dict(vp=8200), -8), (dict(kn=4096), -9), (dict(vn=8192), -9), (dict(vp=4096), -9),
    (dict(H=2 ** 31), -10),
])
def test_append_argument_errors_return_before_any_device_work(kw, code):
    assert _call_append(**kw) == code


def test_empty_append_is_a_no_op():
    assert _call_append(R=0, kn=0, vn=0, kp=0, vp=0, bt=0) == 0


def _call_varlen(**kw):
    a = dict(q=16, kp=16, vp=16, bt=16, stride=8, cu=32, hist=48, n=3, total=12, maxr=6, maxc=100, hq=4, hkv=2,
             d=64, ps=16, S=0, out=4096, dt=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return pkg.lib().paged_prefill_attention_varlen(
        vp(a["q"]), vp(a["kp"]), vp(a["vp"]), vp(a["bt"]), a["stride"], vp(a["cu"]), vp(a["hist"]), a["n"],
        a["total"], a["maxr"], a["maxc"], a["hq"], a["hkv"], a["d"], a["ps"], a["S"], vp(a["out"]), a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), -4), (dict(n=-1), -2), (dict(total=-1), -2), (dict(maxr=13), -2), (dict(maxc=5), -2),
    (dict(stride=6), -2), (dict(S=-1), -2), (dict(n=70000), -10), (dict(d=96), -3), (dict(ps=12), -3),
    (dict(hq=5), -2), (dict(q=0), -1), (dict(bt=0), -1), (dict(cu=0), -1), (dict(hist=0), -1), (dict(out=0), -1),
    (dict(q=24), -8), (dict(out=16 + 64), -9), (dict(maxc=2 ** 31), -10),
])
def test_varlen_argument_errors_return_before_any_device_work(kw, code):
    assert _call_varlen(**kw) == code


def test_empty_varlen_batches_are_no_ops():
    assert _call_varlen(n=0, q=0, kp=0, vp=0, bt=0, cu=0, hist=0, out=0) == 0
    assert _call_varlen(total=0, maxr=0, q=0, kp=0, vp=0, bt=0, cu=0, hist=0, out=0) == 0


def _call_varlen_q8(**kw):
    a = dict(q=16, kq=32, ks=48, vq=64, vs=80, bt=96, stride=8, cu=112, hist=128, n=3, total=12, maxr=6, maxc=100,
             hq=4, hkv=2, d=64, ps=16, S=0, out=8192, dt=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return pkg.lib().paged_prefill_attention_varlen_q8(
        vp(a["q"]), vp(a["kq"]), vp(a["ks"]), vp(a["vq"]), vp(a["vs"]), vp(a["bt"]), a["stride"], vp(a["cu"]),
        vp(a["hist"]), a["n"], a["total"], a["maxr"], a["maxc"], a["hq"], a["hkv"], a["d"], a["ps"], a["S"],
        vp(a["out"]), a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), -4), (dict(n=-1), -2), (dict(maxr=13), -2), (dict(maxc=5), -2), (dict(stride=6), -2),
    (dict(S=-1), -2), (dict(d=96), -3), (dict(ps=8), -3), (dict(ps=1), -3), (dict(ps=12), -3), (dict(hq=5), -2),
    (dict(q=0), -1), (dict(kq=0), -1), (dict(ks=0), -1), (dict(vs=0), -1), (dict(bt=0), -1), (dict(cu=0), -1),
    (dict(out=0), -1), (dict(ks=50), -8), (dict(vq=72), -8), (dict(out=16 + 64), -9), (dict(n=70000), -10),
])
def test_varlen_q8_argument_errors_return_before_any_device_work(kw, code):
    assert _call_varlen_q8(**kw) == code


def test_empty_varlen_q8_batches_are_no_ops():
    nulls = dict(q=0, kq=0, ks=0, vq=0, vs=0, bt=0, cu=0, hist=0, out=0)
    assert _call_varlen_q8(n=0, **nulls) == 0
    assert _call_varlen_q8(total=0, maxr=0, **nulls) == 0


@pytest.mark.parametrize("n,total,max_rows,max_ctx,hq,hkv,d,ps,req", [
    (32, 32, 1, 32769, 16, 2, 256, 16, 0), (8, 2048, 256, 65792, 32, 4, 128, 16, 0), (5, 383, 200, 5016, 8, 2, 128, 16, 3),
    (3, 73, 50, 1000, 4, 1, 64, 8, 0), (2, 40, 33, 433, 2, 2, 256, 32, 500), (1, 1, 1, 1, 4, 1, 64, 1, 0),
])
def test_varlen_plan_invariants(n, total, max_rows, max_ctx, hq, hkv, d, ps, req):
    _check_varlen_plan(n, total, max_rows, max_ctx, hq, hkv, d, ps, req,
                       pkg.paged_prefill_plan_varlen(n, total, max_rows, max_ctx, hq, hkv, d, ps, req))


def _check_varlen_plan(n, total, max_rows, max_ctx, hq, hkv, d, ps, req, p):
    """The documented shape of a varlen plan."""
    g = hq // hkv
    narrow = max_rows * g <= 16 and ps >= 8
    assert (p["m_tile"] == 32) == narrow
    assert p["tiles_m"] == -(-max_rows * g // p["m_tile"])
    assert p["grid"] == n * p["tiles_m"] * hkv * p["n_splits"]
    assert p["n_splits"] * p["split_tokens"] >= max_ctx > (p["n_splits"] - 1) * p["split_tokens"]
    if narrow:
        # a batch of decode steps: one workgroup per CU over the sequences that
        # can have rows and the KV heads, unless the page registers (128 pages
        # per split) ask for more splits
        assert p["split_tokens"] % max(32, ps) == 0 and p["split_tokens"] // ps <= 128
        busy = min(n, total)
        if req == 0 and p["split_tokens"] < 128 * ps:
            assert p["n_splits"] <= max(1, -(-256 // (busy * hkv)))
    else:
        assert p["split_tokens"] % max(64, ps) == 0
    if req == 0 and not narrow:
        # the split rule counts at least one m tile per sequence: a batch of
        # decode rows does not get a one-sequence split count
        tiles = max(-(-total * g // p["m_tile"]), min(n, total))
        assert p["n_splits"] <= max(1, (256 // hkv) // tiles)
    if p["n_splits"] > 1:
        assert p["workspace_bytes"] >= p["n_splits"] * total * hq * (d + 1) * 4
        assert p["merge_grid"] == -(-max_rows * hq // _merge_pairs_per_block(d, p["n_splits"])) * n
    else:
        assert p["workspace_bytes"] == 0 and p["merge_grid"] == 0


@settings(max_examples=300, deadline=None, derandomize=True, database=None)
@given(seqs=st.lists(st.tuples(st.integers(0, 1 << 16), st.integers(0, 300)), min_size=1, max_size=16),
       hkv=st.sampled_from([1, 2, 4, 8]), g=st.sampled_from([1, 2, 4, 8]), d=st.sampled_from([64, 128, 256]),
       ps=st.sampled_from(PS), req=st.one_of(st.just(0), st.integers(1, 64)))
def test_varlen_plan_invariants_random(seqs, hkv, g, d, ps, req):
    """The same over random batches (up to 16 sequences, histories up to 64K,
    0-300 rows each, at least one row in the batch)."""
    if all(r == 0 for _, r in seqs):
        seqs = seqs[:-1] + [(seqs[-1][0], 1)]
    n, total = len(seqs), sum(r for _, r in seqs)
    max_rows, max_ctx = max(r for _, r in seqs), max(h + r for h, r in seqs)
    hq = hkv * g
    try:
        p = pkg.paged_prefill_plan_varlen(n, total, max_rows, max_ctx, hq, hkv, d, ps, req)
    except pkg.PagedPrefillError as e:
        assert e.code in (-5, -10) and req > 0, e   # a requested count past the workspace limits
        return
    _check_varlen_plan(n, total, max_rows, max_ctx, hq, hkv, d, ps, req, p)


def test_varlen_plan_of_one_sequence_is_the_single_call_plan():
    for h, r in ((32768, 2048), (65536, 256), (131072, 128), (1000, 77)):
        a = pkg.paged_prefill_plan(h, r, 16, 2, 256)
        b = pkg.paged_prefill_plan_varlen(1, r, r, h + r, 16, 2, 256)
        assert a == b, (h, r, a, b)


def _call_q8(**kw):
    a = dict(q=16, kq=32, ks=48, vq=64, vs=80, bt=96, H=10, R=4, P=0, hq=4, hkv=2, d=64, ps=16, S=0, out=4096, dt=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return pkg.lib().paged_prefill_attention_q8(
        vp(a["q"]), vp(a["kq"]), vp(a["ks"]), vp(a["vq"]), vp(a["vs"]), vp(a["bt"]), a["H"], a["R"], a["P"], a["hq"],
        a["hkv"], a["d"], a["ps"], a["S"], vp(a["out"]), a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), -4), (dict(R=-1), -2), (dict(H=-1), -2), (dict(d=96), -3), (dict(ps=8), -3), (dict(ps=1), -3),
    (dict(ps=12), -3), (dict(S=-1), -2), (dict(P=-1), -2), (dict(q=0), -1), (dict(ks=0), -1), (dict(vs=0), -1),
    (dict(bt=0), -1), (dict(ks=50), -8), (dict(vq=72), -8), (dict(out=16 + 64), -9),
])
def test_q8_argument_errors_return_before_any_device_work(kw, code):
    assert _call_q8(**kw) == code


def test_empty_q8_chunk_is_a_no_op():
    assert _call_q8(R=0, q=0, kq=0, ks=0, vq=0, vs=0, bt=0, out=0) == 0


def _call_append_q8(**kw):
    a = dict(kn=16, vn=32, kq=4096, ks=8192, vq=12288, vs=16384, bt=64, H=10, R=4, hkv=2, d=64, ps=16, dt=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return pkg.lib().paged_kv_append_q8(vp(a["kn"]), vp(a["vn"]), vp(a["kq"]), vp(a["ks"]), vp(a["vq"]), vp(a["vs"]),
                                        vp(a["bt"]), a["H"], a["R"], a["hkv"], a["d"], a["ps"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), -4), (dict(R=-1), -2), (dict(d=32), -3), (dict(ps=3), -3), (dict(kn=0), -1), (dict(vs=0), -1),
    (dict(bt=0), -1), (dict(ks=8200), -8), (dict(kq=8192), -9), (dict(vs=16), -9),
])
def test_append_q8_argument_errors_return_before_any_device_work(kw, code):
    assert _call_append_q8(**kw) == code


def test_empty_q8_append_is_a_no_op():
    assert _call_append_q8(R=0, kn=0, vn=0, kq=0, ks=0, vq=0, vs=0, bt=0) == 0


def test_binding_rejects_mixed_types_and_shapes_before_any_call():
    """Element types and shapes the C ABI cannot see are checked in the
    binding, on the host, before the library is called."""
    import torch
    import paged_kv_prefill_amd as pkg
    q = torch.zeros(4, 8, 64, dtype=torch.float16)
    kp = torch.zeros(3, 16, 2, 64, dtype=torch.float16)
    bt = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(TypeError):
        pkg.paged_prefill_attention(q, kp.to(torch.bfloat16), kp, bt, 10)
    with pytest.raises(TypeError):
        pkg.paged_prefill_attention(q, kp, kp, bt.to(torch.int64), 10)
    with pytest.raises(ValueError):
        pkg.paged_prefill_attention(q, kp, kp, bt, 10, out=torch.zeros(4, 8, 32, dtype=torch.float16))
    with pytest.raises(ValueError):
        pkg.paged_prefill_attention(q, kp, kp, bt, 10, out=q.to(torch.bfloat16))
    with pytest.raises(TypeError):
        pkg.paged_prefill_attention(q.float(), kp.float(), kp.float(), bt, 10)
    with pytest.raises(TypeError):
        pkg.contiguous_prefill_attention(q, torch.zeros(20, 2, 64, dtype=torch.bfloat16),
                                         torch.zeros(20, 2, 64, dtype=torch.bfloat16), 10)
    with pytest.raises(TypeError):
        pkg.paged_kv_append(torch.zeros(2, 2, 64, dtype=torch.float16), torch.zeros(2, 2, 64, dtype=torch.float16),
                            kp.to(torch.bfloat16), kp.to(torch.bfloat16), bt, 10)
    with pytest.raises(TypeError):
        pkg.paged_prefill_attention_varlen(q, kp, kp, bt.view(1, 3), torch.tensor([0, 4], dtype=torch.int32),
                                           torch.tensor([10], dtype=torch.int32), 4, 14)


def test_binding_rejects_short_block_tables_before_any_call():
    """A block table with fewer than ceil((H + R) / page_size) entries is
    rejected in the binding (the kernels would read past it), on the host,
    for the attention, the 8-bit attention and both appends."""
    import torch
    import paged_kv_prefill_amd as pkg
    q = torch.zeros(4, 8, 64, dtype=torch.float16)          # R = 4
    kp = torch.zeros(6, 16, 2, 64, dtype=torch.float16)     # pages of 16
    short = torch.zeros(1, dtype=torch.int32)               # H + R = 20 tokens need 2 pages
    with pytest.raises(ValueError, match="need 2 pages"):
        pkg.paged_prefill_attention(q, kp, kp, short, 16)
    with pytest.raises(ValueError, match="need 2 pages"):
        pkg.paged_prefill_attention(q, kp, kp, short, 16, piece_rows=2)
    kq = torch.zeros(6, 16, 2, 64, dtype=torch.int8)
    ks = torch.zeros(6, 16, 2, 2, dtype=torch.float16)
    with pytest.raises(ValueError, match="need 2 pages"):
        pkg.paged_prefill_attention_q8(q, kq, ks, kq, ks, short, 16)
    kn = torch.zeros(4, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="need 2 pages"):
        pkg.paged_kv_append(kn, kn, kp, kp.clone(), short, 16)
    with pytest.raises(ValueError, match="need 2 pages"):
        pkg.paged_kv_append_q8(kn, kn, kq, ks, kq.clone(), ks.clone(), short, 16)
    # a table just long enough passes this check (and stops at the next one: CPU tensors)
    ok = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="on the GPU"):
        pkg.paged_prefill_attention(q, kp, kp, ok, 16)
