"""Seeded random shapes through the C ABI against the fp64 oracle: history,
rows, head counts, head dimension, page size, element type, split request,
piece size and table kind drawn together, so that combinations no
hand-written case names (a ragged last tile in a split that also holds the
causal edge, tiny pages with many splits, pieces over scattered pages) meet
the parity bar.  Paged equals contiguous bit for bit where both use the same
plan (pages of at most 64 tokens).  The same for packed varlen batches and
for 8-bit pages."""

import numpy as np
import pytest

import _gpu
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

N_CASES = 40


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    ps = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256]))
    history = int(rng.choice([0, rng.integers(1, 64), rng.integers(64, 1500)]))
    rows = int(rng.choice([1, rng.integers(2, 33), rng.integers(33, 140)]))
    dtype = str(rng.choice(["f16", "bf16"]))
    n_splits = int(rng.choice([0, 0, 1, 2, 5, 16, 40]))
    table = str(rng.choice(["permute", "scatter"]))
    piece = int(rng.choice([0, 0, 0, rng.integers(1, max(2, rows))]))
    return dict(i=i, d=d, hkv=hkv, hq=hkv * g, ps=ps, history=history, rows=rows, dtype=dtype,
                n_splits=n_splits, table=table, piece=piece if piece < rows else 0)


CASES = [_draw(i) for i in range(N_CASES)]


def _id(c):
    return f"H{c['history']}-R{c['rows']}-{c['hq']}x{c['hkv']}-d{c['d']}-ps{c['ps']}-{c['dtype']}-S{c['n_splits']}" \
           f"-{c['table']}" + (f"-p{c['piece']}" if c["piece"] else "")


def _same_plans(c):
    """Paged and contiguous calls run the same launches (so agree bit for bit)
    when every call (each piece, or the whole chunk) gets the same plan: the
    contiguous entry plans as for pages of 16 tokens."""
    step = c["piece"] or c["rows"]
    for r0 in range(0, c["rows"], step):
        r = min(step, c["rows"] - r0)
        args = (c["history"] + r0, r, c["hq"], c["hkv"], c["d"])
        if pkg.paged_prefill_plan(*args, c["ps"], c["n_splits"]) != pkg.paged_prefill_plan(*args, 16, c["n_splits"]):
            return False
    return True


@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_matches_oracle(c):
    import torch
    ctx = c["history"] + c["rows"]
    n_pages = -(-ctx // c["ps"])
    pool = n_pages + 7 if c["table"] == "scatter" else None
    case = synth.make_case("random", c["history"], c["rows"], c["hq"], c["hkv"], c["d"], c["ps"], c["dtype"],
                           seed=2000 + c["i"], table=c["table"], pool_pages=pool)
    print(f"case random {_id(c)}", flush=True)
    d = _gpu.dev_case(case)
    out = pkg.paged_prefill_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], c["history"],
                                      n_splits=c["n_splits"], piece_rows=c["piece"])
    out_c = pkg.contiguous_prefill_attention(d["q"], d["k"], d["v"], c["history"], n_splits=c["n_splits"],
                                             piece_rows=c["piece"])
    torch.cuda.synchronize()
    if _same_plans(c):
        assert _gpu.bits_equal(out, out_c), "paged and contiguous differ bitwise"
    got = _gpu.host_out(out)
    ref = _gpu.oracle_out(case)
    if c["dtype"] == "f16":
        _gpu.assert_close(got, ref, _id(c))
    else:
        _gpu.assert_close_bf16_bound(got, ref, _gpu.oracle_abs_weighted(case), _id(c))


def _draw_varlen(i):
    rng = np.random.default_rng(3000 + i)
    n = int(rng.integers(1, 9))
    seqs = []
    for _ in range(n):
        h = int(rng.choice([0, rng.integers(1, 100), rng.integers(100, 2000)]))
        r = int(rng.choice([0, 1, rng.integers(2, 40), rng.integers(40, 200)]))
        seqs.append((h, r))
    if all(r == 0 for _, r in seqs):
        seqs[0] = (seqs[0][0], 1)
    hkv = int(rng.choice([1, 2, 4]))
    return dict(i=i, seqs=seqs, hkv=hkv, hq=hkv * int(rng.choice([1, 2, 4, 8])), d=int(rng.choice([64, 128, 256])),
                ps=int(rng.choice([1, 4, 8, 16, 32, 128])), dtype=str(rng.choice(["f16", "bf16"])),
                n_splits=int(rng.choice([0, 0, 1, 3, 17])))


VARLEN = [_draw_varlen(i) for i in range(12)]


def _vid(c):
    return f"n{len(c['seqs'])}-{c['hq']}x{c['hkv']}-d{c['d']}-ps{c['ps']}-{c['dtype']}-S{c['n_splits']}"


@pytest.mark.parametrize("c", VARLEN, ids=[_vid(c) for c in VARLEN])
def test_random_varlen_batch_matches_oracle(c):
    import torch
    import oracle
    case = synth.make_varlen_case("random_varlen", c["seqs"], c["hq"], c["hkv"], c["d"], c["ps"], c["dtype"],
                                  seed=4000 + c["i"])
    print(f"case random varlen {_vid(c)}: {c['seqs']}", flush=True)
    dt = _gpu.torch_dtype(c["dtype"])
    dev = "cuda:0"
    out = pkg.paged_prefill_attention_varlen(
        _gpu.to_dev(case.q, dt), _gpu.to_dev(case.k_pages, dt), _gpu.to_dev(case.v_pages, dt),
        torch.from_numpy(case.block_tables).to(dev), torch.from_numpy(case.cu_rows).to(dev),
        torch.from_numpy(case.history_lens).to(dev), case.max_rows, case.max_context, n_splits=c["n_splits"])
    torch.cuda.synchronize()
    if int(case.cu_rows[-1]) == 0:
        return
    dec = oracle.decode_f16 if c["dtype"] == "f16" else oracle.decode_bf16
    ref = oracle.varlen_paged_attention(dec(case.q), dec(case.k_pages), dec(case.v_pages), case.block_tables,
                                        case.cu_rows, case.history_lens, case.page_size)
    got = _gpu.host_out(out)
    # the tolerance holds per sequence (each sequence's rows are their own attention output)
    for s in range(len(c["seqs"])):
        r0, r1 = int(case.cu_rows[s]), int(case.cu_rows[s + 1])
        if r1 == r0:
            continue
        what = f"{_vid(c)} sequence {s} {c['seqs'][s]}"
        if c["dtype"] == "f16":
            _gpu.assert_close(got[r0:r1], ref[r0:r1], what)
        else:
            absw = oracle.varlen_paged_attention(dec(case.q), dec(case.k_pages), np.abs(dec(case.v_pages)),
                                                 case.block_tables, case.cu_rows, case.history_lens,
                                                 case.page_size)
            _gpu.assert_close_bf16_bound(got[r0:r1], ref[r0:r1], absw[r0:r1], what)


def _draw_q8(i):
    rng = np.random.default_rng(5000 + i)
    hkv = int(rng.choice([1, 2, 4]))
    return dict(i=i, history=int(rng.choice([0, rng.integers(1, 100), rng.integers(100, 2500)])),
                rows=int(rng.choice([1, rng.integers(2, 40), rng.integers(40, 160)])), hkv=hkv,
                hq=hkv * int(rng.choice([1, 2, 4, 8])), d=int(rng.choice([64, 128, 256])),
                ps=int(rng.choice([16, 32, 64, 128, 256])), dtype=str(rng.choice(["f16", "bf16"])),
                n_splits=int(rng.choice([0, 0, 1, 3, 17])))


Q8 = [_draw_q8(i) for i in range(12)]


def _qid(c):
    return f"H{c['history']}-R{c['rows']}-{c['hq']}x{c['hkv']}-d{c['d']}-ps{c['ps']}-{c['dtype']}-S{c['n_splits']}"


@pytest.mark.parametrize("c", Q8, ids=[_qid(c) for c in Q8])
def test_random_q8_shape_matches_oracle(c):
    import torch
    import oracle
    case = synth.make_q8_case("random_q8", c["history"], c["rows"], c["hq"], c["hkv"], c["d"], c["ps"], c["dtype"],
                              seed=6000 + c["i"])
    print(f"case random q8 {_qid(c)}", flush=True)
    dev = "cuda:0"
    q = _gpu.to_dev(case.q, _gpu.torch_dtype(c["dtype"]))
    t = [torch.from_numpy(a).to(dev) for a in (case.k_quant, case.k_scale.view(np.int16), case.v_quant,
                                               case.v_scale.view(np.int16), case.block_table)]
    out = pkg.paged_prefill_attention_q8(q, t[0], t[1], t[2], t[3], t[4], c["history"], n_splits=c["n_splits"])
    torch.cuda.synchronize()
    dec = oracle.decode_f16 if c["dtype"] == "f16" else oracle.decode_bf16
    ks, vs = oracle.decode_scales(case.k_scale), oracle.decode_scales(case.v_scale)
    ref = oracle.paged_q8_attention(dec(case.q), case.k_quant, ks, case.v_quant, vs, case.block_table,
                                    c["history"], c["ps"])
    got = _gpu.host_out(out)
    if c["dtype"] == "f16":
        _gpu.assert_close(got, ref, _qid(c))
    else:
        # sum_j p_j |V_j| with |V| = |scale| |quant|
        absw = oracle.paged_q8_attention(dec(case.q), case.k_quant, ks, np.abs(case.v_quant), np.abs(vs),
                                         case.block_table, c["history"], c["ps"])
        _gpu.assert_close_bf16_bound(got, ref, absw, _qid(c))
