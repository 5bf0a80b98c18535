"""The opt-in host checks (PPA_VALIDATE=1), through the C ABI: a paged call,
a call over 8-bit pages, varlen batches over 16-bit and 8-bit pages and both
appends copy their device
arrays to the host first and return PPA_ERR_BLOCK_TABLE for a negative
block-table entry, PPA_ERR_BAD_SHAPE for varlen arrays that break the
host-side bounds, before any launch (the output, or the pool an append
writes, is left as it was); valid calls give the same bits as without the
checks.  Every pool here sits inside a larger allocation with pages of slack
on both sides, and every table row is long enough for its sequence, so a bad
call stays inside allocated memory even if a check let it through."""

import numpy as np
import pytest

import _gpu
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ERR_BAD_SHAPE, ERR_BLOCK_TABLE = -2, -7
SLACK = 4   # pages of slack before and after each pool


def _padded(t):
    """t [n][...] as a view into an allocation with SLACK leading and trailing
    entries (filled with -1 bits: NaN for 16-bit values, NaN scales)."""
    import torch
    big = torch.full((t.shape[0] + 2 * SLACK,) + tuple(t.shape[1:]), -1, dtype=t.dtype, device=t.device)
    big[SLACK:SLACK + t.shape[0]] = t
    return big[SLACK:SLACK + t.shape[0]]


def _expect(code, fn, *watched):
    """fn() raises the library error `code`, and the watched tensors keep
    their bits (nothing was launched)."""
    import torch
    before = [w.clone() for w in watched]
    with pytest.raises(pkg.PagedPrefillError) as e:
        fn()
    torch.cuda.synchronize()
    assert e.value.code == code, e.value
    for w, b in zip(watched, before):
        assert torch.equal(w.view(torch.uint8) if w.dtype != torch.uint8 else w,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def _paged_case():
    case = synth.make_case("validate", 300, 5, 8, 2, 64, 16, "f16", seed=3)
    d = _gpu.dev_case(case, contiguous=False)
    d["k_pages"], d["v_pages"] = _padded(d["k_pages"]), _padded(d["v_pages"])
    return case, d


def test_paged_call_checks_its_table(monkeypatch):
    import torch
    case, d = _paged_case()
    print("case validate paged", flush=True)
    ref = pkg.paged_prefill_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], case.history)
    monkeypatch.setenv("PPA_VALIDATE", "1")
    got = pkg.paged_prefill_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], case.history)
    torch.cuda.synchronize()
    assert _gpu.bits_equal(got, ref)
    bad = d["block_table"].clone()
    bad[3] = -1
    out = torch.full_like(d["q"], 7.0)
    for piece_rows in (0, 2):
        _expect(ERR_BLOCK_TABLE, lambda: pkg.paged_prefill_attention(d["q"], d["k_pages"], d["v_pages"], bad,
                                                                     case.history, out=out, piece_rows=piece_rows),
                out)


def test_q8_call_checks_its_table(monkeypatch):
    import torch
    case = synth.make_q8_case("validate_q8", 300, 5, 8, 2, 64, 16, "f16", seed=4)
    dev = "cuda:0"
    q = _gpu.to_dev(case.q, torch.float16)
    kq, vq = _padded(torch.from_numpy(case.k_quant).to(dev)), _padded(torch.from_numpy(case.v_quant).to(dev))
    ks = _padded(torch.from_numpy(case.k_scale.view(np.int16)).to(dev))
    vs = _padded(torch.from_numpy(case.v_scale.view(np.int16)).to(dev))
    bt = torch.from_numpy(case.block_table).to(dev)
    print("case validate q8", flush=True)
    ref = pkg.paged_prefill_attention_q8(q, kq, ks, vq, vs, bt, case.history)
    monkeypatch.setenv("PPA_VALIDATE", "1")
    got = pkg.paged_prefill_attention_q8(q, kq, ks, vq, vs, bt, case.history)
    torch.cuda.synchronize()
    assert _gpu.bits_equal(got, ref)
    bad = bt.clone()
    bad[-1] = -1
    out = torch.full_like(q, 7.0)
    _expect(ERR_BLOCK_TABLE, lambda: pkg.paged_prefill_attention_q8(q, kq, ks, vq, vs, bad, case.history, out=out),
            out)


def test_varlen_checks_its_arrays(monkeypatch):
    import torch
    seqs = [(200, 3), (50, 1), (400, 2)]
    case = synth.make_varlen_case("validate_varlen", seqs, 8, 2, 64, 16, "f16", seed=5)
    dev = "cuda:0"
    q = _gpu.to_dev(case.q, torch.float16)
    kp, vp = _padded(_gpu.to_dev(case.k_pages, torch.float16)), _padded(_gpu.to_dev(case.v_pages, torch.float16))
    bt = torch.from_numpy(case.block_tables).to(dev)
    cu = torch.from_numpy(case.cu_rows).to(dev)
    hist = torch.from_numpy(case.history_lens).to(dev)
    assert bt.shape[1] * 16 >= 402   # every row covers its sequence's context

    def call(bt_=bt, cu_=cu, hist_=hist, max_rows=case.max_rows, max_context=case.max_context, out=None):
        return pkg.paged_prefill_attention_varlen(q, kp, vp, bt_, cu_, hist_, max_rows, max_context, out=out)

    print("case validate varlen", flush=True)
    ref = call()
    monkeypatch.setenv("PPA_VALIDATE", "1")
    got = call()
    torch.cuda.synchronize()
    assert _gpu.bits_equal(got, ref)
    out = torch.full_like(q, 7.0)
    bad_bt = bt.clone()
    bad_bt[1, 2] = -1   # sequence 1's third page (its context has 51 tokens: four pages)
    _expect(ERR_BLOCK_TABLE, lambda: call(bt_=bad_bt, out=out), out)
    # row offsets that do not start at 0 (the rows stay inside q)
    _expect(ERR_BAD_SHAPE, lambda: call(cu_=torch.tensor([1, 3, 4, 6], dtype=torch.int32, device=dev), out=out), out)
    # row offsets that end short of total_rows
    _expect(ERR_BAD_SHAPE, lambda: call(cu_=torch.tensor([0, 3, 4, 5], dtype=torch.int32, device=dev), out=out), out)
    # a sequence with more rows than max_rows
    _expect(ERR_BAD_SHAPE, lambda: call(max_rows=2, out=out), out)
    # a sequence past max_context
    _expect(ERR_BAD_SHAPE, lambda: call(max_context=case.max_context - 1, out=out), out)


def test_appends_check_their_table(monkeypatch):
    import torch
    history, rows, hkv, d, ps = 300, 5, 2, 64, 16
    n_pages = -(-(history + rows) // ps)
    rng = np.random.default_rng(6)
    dev = "cuda:0"
    bt = torch.from_numpy(rng.permutation(n_pages).astype(np.int32)).to(dev)
    bad = bt.clone()
    bad[history // ps] = -1   # the page the first new row goes to
    monkeypatch.setenv("PPA_VALIDATE", "1")
    print("case validate appends", flush=True)
    kn = torch.randn((rows, hkv, d), device=dev).half()
    vn = torch.randn((rows, hkv, d), device=dev).half()
    kp = _padded(torch.zeros((n_pages, ps, hkv, d), dtype=torch.float16, device=dev))
    vp = _padded(torch.zeros((n_pages, ps, hkv, d), dtype=torch.float16, device=dev))
    _expect(ERR_BLOCK_TABLE, lambda: pkg.paged_kv_append(kn, vn, kp, vp, bad, history), kp, vp)
    pkg.paged_kv_append(kn, vn, kp, vp, bt, history)   # the valid table passes the check and writes
    torch.cuda.synchronize()
    pos = history + np.arange(rows)
    pages = torch.from_numpy(bt.cpu().numpy()[pos // ps].astype(np.int64)).to(dev)
    slots = torch.from_numpy((pos % ps).astype(np.int64)).to(dev)
    assert torch.equal(kp[pages, slots], kn) and torch.equal(vp[pages, slots], vn)
    kq = _padded(torch.zeros((n_pages, ps, hkv, d), dtype=torch.int8, device=dev))
    vq = _padded(torch.zeros((n_pages, ps, hkv, d), dtype=torch.int8, device=dev))
    ksc = _padded(torch.zeros((n_pages, ps, hkv, d // 32), dtype=torch.int16, device=dev))
    vsc = _padded(torch.zeros((n_pages, ps, hkv, d // 32), dtype=torch.int16, device=dev))
    _expect(ERR_BLOCK_TABLE, lambda: pkg.paged_kv_append_q8(kn, vn, kq, ksc, vq, vsc, bad, history), kq, vq, ksc, vsc)


def test_varlen_q8_checks_its_arrays(monkeypatch):
    import torch
    seqs = [(200, 3), (50, 1), (400, 2)]
    case = synth.make_varlen_q8_case("validate_varlen_q8", seqs, 8, 2, 64, 16, "f16", seed=7)
    dev = "cuda:0"
    q = _gpu.to_dev(case.q, torch.float16)
    kq, vq = _padded(torch.from_numpy(case.k_quant).to(dev)), _padded(torch.from_numpy(case.v_quant).to(dev))
    ks = _padded(torch.from_numpy(case.k_scale.view(np.int16)).to(dev))
    vs = _padded(torch.from_numpy(case.v_scale.view(np.int16)).to(dev))
    bt = torch.from_numpy(case.block_tables).to(dev)
    cu = torch.from_numpy(case.cu_rows).to(dev)
    hist = torch.from_numpy(case.history_lens).to(dev)

    def call(bt_=bt, max_rows=case.max_rows, out=None):
        return pkg.paged_prefill_attention_varlen_q8(q, kq, ks, vq, vs, bt_, cu, hist, max_rows, case.max_context,
                                                     out=out)

    print("case validate varlen q8", flush=True)
    ref = call()
    monkeypatch.setenv("PPA_VALIDATE", "1")
    got = call()
    torch.cuda.synchronize()
    assert _gpu.bits_equal(got, ref)
    out = torch.full_like(q, 7.0)
    bad_bt = bt.clone()
    bad_bt[2, 5] = -1
    _expect(ERR_BLOCK_TABLE, lambda: call(bt_=bad_bt, out=out), out)
    _expect(ERR_BAD_SHAPE, lambda: call(max_rows=2, out=out), out)
