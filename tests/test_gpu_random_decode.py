"""Seeded random decode-sized calls (few query vectors per KV head) through
the C ABI against the fp64 oracle: history, rows, head counts, head
dimension, page size, element type and split request drawn together, over
16-bit pages (at most 16 query vectors per KV head: the narrow kernel) and
8-bit pages (at most 32), so that combinations the hand-written cases do
not name (a ragged last tile in a split that also holds the causal edge,
large pages with many splits, group sizes with empty MFMA columns) meet
the parity bar."""

import numpy as np
import pytest

import _gpu
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

N16, N8 = 24, 16


def _draw(i, q8):
    rng = np.random.default_rng((2000 if q8 else 3000) + i)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    limit = 32 if q8 else 16
    rows = int(rng.integers(1, max(1, limit // g) + 1))
    ps = int(rng.choice([16, 32, 64, 256, 1024] if q8 else [8, 16, 32, 64, 128, 512]))
    history = int(rng.choice([rng.integers(0, 40), rng.integers(40, 3000), rng.integers(3000, 20000)]))
    dtype = str(rng.choice(["f16", "bf16"]))
    n_splits = int(rng.choice([0, 0, 0, 1, 2, 7, 100000]))
    return dict(i=i, d=d, hkv=hkv, hq=hkv * g, rows=rows, ps=ps, history=history, dtype=dtype, n_splits=n_splits)


CASES16 = [_draw(i, False) for i in range(N16)]
CASES8 = [_draw(i, True) for i in range(N8)]


def _id(c):
    return f"H{c['history']}-R{c['rows']}-{c['hq']}x{c['hkv']}-d{c['d']}-ps{c['ps']}-{c['dtype']}-S{c['n_splits']}"


def _assert(case, got, ref, absw, what):
    if case.dtype == "f16":
        _gpu.assert_close(got, ref, what)
    else:
        _gpu.assert_close_bf16_bound(got, ref, absw, what)


@pytest.mark.parametrize("c", CASES16, ids=[_id(c) for c in CASES16])
def test_random_decode_16bit(c):
    import torch
    plan = pkg.paged_prefill_plan(c["history"], c["rows"], c["hq"], c["hkv"], c["d"], c["ps"], c["n_splits"])
    assert plan["m_tile"] == 32, plan   # every draw is decode-sized
    print(f"case random decode 16-bit {_id(c)}: S={plan['n_splits']}", flush=True)
    case = synth.make_case("rand_dec", c["history"], c["rows"], c["hq"], c["hkv"], c["d"], c["ps"], c["dtype"],
                           seed=c["i"] + 11)
    dev = _gpu.dev_case(case, contiguous=False)
    out = pkg.paged_prefill_attention(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], c["history"],
                                      n_splits=c["n_splits"])
    torch.cuda.synchronize()
    absw = _gpu.oracle_abs_weighted(case) if c["dtype"] == "bf16" else None
    _assert(case, _gpu.host_out(out), _gpu.oracle_out(case), absw, _id(c))


@pytest.mark.parametrize("c", CASES8, ids=[_id(c) for c in CASES8])
def test_random_decode_8bit(c):
    import torch
    from test_gpu_q8 import _dev_q8, _oracle, _oracle_absw, _run
    print(f"case random decode 8-bit {_id(c)}", flush=True)
    case = synth.make_q8_case("rand_dec_q8", c["history"], c["rows"], c["hq"], c["hkv"], c["d"], c["ps"], c["dtype"],
                              seed=c["i"] + 13)
    out = _run(_dev_q8(case), case, n_splits=c["n_splits"])
    torch.cuda.synchronize()
    absw = _oracle_absw(case) if c["dtype"] == "bf16" else None
    _assert(case, _gpu.host_out(out), _oracle(case), absw, _id(c))
