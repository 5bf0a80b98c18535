"""CPU-side checks of the C ABI: the library loads, exports every function
include/paged_prefill.h declares, and its host-only helpers (planner, split
rule, piece rule, block-table check, argument checks) behave as documented.
No call here reaches a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

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
    assert len(names) == 16, names
    for name in names:
        assert hasattr(lib, name), name
    assert lib.paged_prefill_version() == 10000


def test_binding_covers_every_declared_symbol():
    for name in declared_functions():
        assert name in pkg._SIGNATURES, name


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


@pytest.mark.parametrize("history,rows,hq,hkv,d,ps,req", [
    (0, 1, 1, 1, 64, 16, 0), (5, 3, 4, 1, 64, 1, 0), (512, 64, 4, 1, 64, 16, 4), (1000, 77, 6, 2, 128, 8, 0),
    (131072, 128, 16, 2, 256, 16, 0), (100, 2048, 32, 4, 128, 256, 0), (37, 5, 16, 2, 256, 16, 64),
    (8192, 512, 16, 2, 256, 16, 0), (65536, 2048, 32, 8, 128, 16, 0), (3, 1, 2, 2, 64, 1024, 5),
])
def test_plan_invariants(history, rows, hq, hkv, d, ps, req):
    p = pkg.paged_prefill_plan(history, rows, hq, hkv, d, ps, req)
    ctx = history + rows
    unit = max(64, ps)
    assert p["split_tokens"] % 64 == 0 and p["split_tokens"] % ps == 0
    assert 1 <= p["n_splits"] <= 64
    # the splits cover [0, ctx) and none is empty
    assert (p["n_splits"] - 1) * p["split_tokens"] < ctx <= p["n_splits"] * p["split_tokens"]
    # two query blocks per wave (256-vector m tiles) at d <= 128 once the call
    # has more query vectors than one 128-vector tile
    assert p["m_tile"] == (256 if d <= 128 and rows * (hq // hkv) > 128 else 128)
    assert p["tiles_m"] == -(-rows * (hq // hkv) // p["m_tile"])
    assert p["grid"] == p["tiles_m"] * hkv * p["n_splits"]
    if req:
        assert p["n_splits"] <= max(1, min(req, -(-ctx // unit)))
    if p["n_splits"] > 1:
        assert p["workspace_bytes"] >= p["n_splits"] * rows * hq * (d + 1) * 4
        groups = 4 if p["n_splits"] >= 16 else 1
        assert p["merge_grid"] == -(-rows * hq // (256 // (d // 4 * groups)))
    else:
        assert p["workspace_bytes"] == 0 and p["merge_grid"] == 0


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


@pytest.mark.parametrize("n,total,max_rows,max_ctx,hq,hkv,d,ps,req", [
    (32, 32, 1, 32769, 16, 2, 256, 16, 0), (8, 2048, 256, 65792, 32, 4, 128, 16, 0), (5, 383, 200, 5016, 8, 2, 128, 16, 3),
    (3, 73, 50, 1000, 4, 1, 64, 8, 0), (2, 40, 33, 433, 2, 2, 256, 32, 500), (1, 1, 1, 1, 4, 1, 64, 1, 0),
])
def test_varlen_plan_invariants(n, total, max_rows, max_ctx, hq, hkv, d, ps, req):
    p = pkg.paged_prefill_plan_varlen(n, total, max_rows, max_ctx, hq, hkv, d, ps, req)
    g = hq // hkv
    assert p["tiles_m"] == -(-max_rows * g // p["m_tile"])
    assert p["grid"] == n * p["tiles_m"] * hkv * p["n_splits"]
    assert p["split_tokens"] % max(64, ps) == 0
    assert p["n_splits"] * p["split_tokens"] >= max_ctx > (p["n_splits"] - 1) * p["split_tokens"]
    if req == 0:
        # the split rule counts at least one m tile per sequence: a batch of
        # decode rows does not get a one-sequence split count
        tiles = max(-(-total * g // p["m_tile"]), min(n, total))
        assert p["n_splits"] <= max(1, (256 // hkv) // tiles)
    if p["n_splits"] > 1:
        assert p["workspace_bytes"] >= p["n_splits"] * total * hq * (d + 1) * 4
        groups = 4 if p["n_splits"] >= 16 else 1
        assert p["merge_grid"] == -(-max_rows * hq // (256 // (d // 4 * groups))) * n
    else:
        assert p["workspace_bytes"] == 0 and p["merge_grid"] == 0


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
