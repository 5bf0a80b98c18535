"""Seeded random shapes through the C ABI against the fp64 oracle: history,
rows, head counts, head dimension, page size, element type, split request,
piece size and table kind drawn together, so that combinations no
hand-written case names (a ragged last tile in a split that also holds the
causal edge, tiny pages with many splits, pieces over scattered pages) meet
the parity bar.  Paged equals contiguous bit for bit where both use the same
plan (pages of at most 64 tokens)."""

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
    if c["ps"] <= 64:
        assert _gpu.bits_equal(out, out_c), "paged and contiguous differ bitwise"
    got = _gpu.host_out(out)
    ref = _gpu.oracle_out(case)
    if c["dtype"] == "f16":
        _gpu.assert_close(got, ref, _id(c))
    else:
        _gpu.assert_close_bf16_bound(got, ref, _gpu.oracle_abs_weighted(case), _id(c))
