"""The narrow kernel (decode steps and appends of few query vectors per KV
head: at most 16 over 16-bit K/V, 32 over 8-bit pages) through the C ABI
against the fp64 oracle: head dimensions 64, 128 and 256, fp16 and bf16,
16-bit pages of 8 to 1024 tokens, contiguous K/V and 8-bit pages; split
counts from one to one 32-key tile per split; contexts shorter than a tile,
ragged tails and workgroups whose waves have no tile; score outliers that
make a wave raise its softmax reference.  Paged and contiguous results agree
bit for bit where both get the same plan (the same kernel, addressing
aside).  The 16-bit cases
of 17-32 query vectors run the prefill kernel (faster there) and are held to
the same bar."""

import numpy as np
import pytest

import _gpu
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

# name, history, rows, Hq, Hkv, d, ps, dtype, n_splits
CASES = [
    ("d128_1row", 5000, 1, 32, 4, 128, 16, "f16", 0),
    ("d256_1row", 7000, 1, 16, 2, 256, 16, "bf16", 0),
    ("d64_g32", 3000, 1, 32, 1, 64, 8, "f16", 0),            # 32 query vectors of one row
    ("d128_4rows_ps32", 2500, 4, 16, 2, 128, 32, "bf16", 0),  # 4 rows x 8 heads
    ("d256_2rows_ps64", 1900, 2, 32, 2, 256, 64, "f16", 0),   # 2 rows x 16 heads
    ("d64_tiny", 5, 1, 4, 1, 64, 8, "f16", 0),                # 6 keys: less than a tile
    ("d128_ctx33", 32, 1, 8, 2, 128, 16, "f16", 0),          # one tile and one key
    ("d256_one_split", 3333, 3, 16, 2, 256, 16, "f16", 1),    # many tiles per wave
    ("d128_tile_splits", 4000, 1, 8, 1, 128, 16, "bf16", 100000),  # one tile per split
    ("d64_ps256", 10000, 2, 16, 2, 64, 256, "f16", 0),
    ("d256_ps8_S5", 2049, 1, 8, 1, 256, 8, "bf16", 5),
    ("d128_rows_past_group", 600, 32, 1, 1, 128, 16, "f16", 0),  # 32 rows, one head: causal inside
    ("d128_ps512", 3000, 1, 16, 2, 128, 512, "bf16", 0),     # several tiles per page
    ("d256_ps1024_S3", 2500, 2, 16, 2, 256, 1024, "f16", 3),  # the largest pages, one per split
    ("d128_hkv16", 8000, 1, 128, 16, 128, 16, "bf16", 0),     # many KV heads: 16 splits per head
    ("d64_mha32", 3000, 4, 32, 32, 64, 16, "f16", 0),         # no grouping: 4 query vectors per KV head
]


def _check(case, out, what):
    got = _gpu.host_out(out)
    ref = _gpu.oracle_out(case)
    if case.dtype == "f16":
        _gpu.assert_close(got, ref, what)
    else:
        _gpu.assert_close_bf16_bound(got, ref, _gpu.oracle_abs_weighted(case), what)


@pytest.mark.parametrize("name,history,rows,hq,hkv,d,ps,dtype,n_splits", CASES, ids=[c[0] for c in CASES])
def test_narrow_matches_oracle(name, history, rows, hq, hkv, d, ps, dtype, n_splits):
    import torch
    plan = pkg.paged_prefill_plan(history, rows, hq, hkv, d, ps, n_splits)
    assert (plan["m_tile"] == 32) == (rows * hq // hkv <= 16), plan
    print(f"case narrow {name}: H={history} R={rows} {hq}/{hkv} d={d} ps={ps} {dtype} S={plan['n_splits']} "
          f"grid={plan['grid']}", flush=True)
    case = synth.make_case(name, history, rows, hq, hkv, d, ps, dtype, seed=history + 7 * rows + d)
    dev = _gpu.dev_case(case)
    out = pkg.paged_prefill_attention(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], history,
                                      n_splits=n_splits)
    out_c = pkg.contiguous_prefill_attention(dev["q"], dev["k"], dev["v"], history, n_splits=n_splits)
    torch.cuda.synchronize()
    # the contiguous entry plans as for pages of 16 tokens: with the same plan
    # the results agree bit for bit, otherwise each meets the oracle
    if pkg.paged_prefill_plan(history, rows, hq, hkv, d, 16, n_splits) == plan:
        assert _gpu.bits_equal(out, out_c), "paged and contiguous differ bitwise"
    else:
        _check(case, out_c, f"{name} contiguous")
    _check(case, out, f"{name} S={plan['n_splits']}")


@pytest.mark.parametrize("n_splits", [1, 3, 17, 0])
def test_narrow_split_count_changes_rounding_only(n_splits):
    """The same decode step under several split counts: each within the
    tolerance of the oracle (the splits only change fp32 summation order)."""
    import torch
    case = synth.make_case("split_inv", 9000, 2, 16, 2, 128, 16, "f16", seed=5)
    dev = _gpu.dev_case(case, contiguous=False)
    out = pkg.paged_prefill_attention(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], case.history,
                                      n_splits=n_splits)
    torch.cuda.synchronize()
    _check(case, out, f"S={n_splits}")


# where the planted key sits, its K[., 0] value: see test_gpu_parity's outlier
# test (q[., 0] + 2, so the key scores about 0.255 value log2 units above the
# rest at d 128): 80 overflows fp16 weights, 300 the bf16 sum bound.
OUTLIERS = [("late", 80.0), ("early", 80.0), ("late", 300.0), ("two_late", 300.0)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("where,value", OUTLIERS, ids=[f"{w}-{int(v)}" for w, v in OUTLIERS])
def test_narrow_score_outliers(dtype, where, value):
    """A key that scores far above a wave's first tile makes that wave raise
    its reference and rescale; the waves' references then differ and the
    workgroup combines them by exact powers of two.  At the planner's split
    count each wave of this shape streams one tile (the outlier sets that
    wave's first reference); with one split requested (two here: a split
    holds at most 128 pages) every wave streams eight, so a late outlier
    arrives after its first."""
    import torch
    from test_gpu_parity import _plant_outlier
    case = synth.make_case("narrow_outlier", 3000, 2, 16, 2, 128, 16, dtype, seed=31)
    keys = {"late": [2900], "early": [40], "two_late": [2500, 2950]}[where]
    for i, key in enumerate(keys):
        case = _plant_outlier(case, key, value * (1 + 0.1 * i), shift_q=(i == 0))
    dev = _gpu.dev_case(case, contiguous=False)
    for s in (0, 1):
        print(f"case narrow outlier {dtype} {where} {value} S={s}", flush=True)
        out = pkg.paged_prefill_attention(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                                          case.history, n_splits=s)
        torch.cuda.synchronize()
        assert np.all(np.isfinite(_gpu.host_out(out)))
        _check(case, out, f"outlier {where} {value} S={s}")


# 8-bit pages (pages of >= 16 tokens): name, history, rows, Hq, Hkv, d, ps, dtype, n_splits
Q8_CASES = [
    ("q8_d256_1row", 6000, 1, 16, 2, 256, 16, "bf16", 0),
    ("q8_d128_4rows_ps32", 3000, 4, 32, 4, 128, 32, "f16", 0),
    ("q8_d64_g32", 2000, 1, 32, 1, 64, 16, "f16", 0),
    ("q8_d64_ps64_S3", 77, 2, 8, 1, 64, 64, "bf16", 3),
    ("q8_d256_tiny", 3, 1, 8, 1, 256, 16, "f16", 0),
    ("q8_d128_one_split", 2500, 1, 16, 2, 128, 16, "bf16", 1),
    ("q8_d256_tile_splits", 1500, 2, 16, 1, 256, 16, "f16", 100000),
    ("q8_d128_ps1024", 2200, 1, 16, 2, 128, 1024, "bf16", 0),
]


@pytest.mark.parametrize("name,history,rows,hq,hkv,d,ps,dtype,n_splits", Q8_CASES, ids=[c[0] for c in Q8_CASES])
def test_narrow_q8_matches_oracle(name, history, rows, hq, hkv, d, ps, dtype, n_splits):
    import torch
    from test_gpu_q8 import _dev_q8, _oracle, _oracle_absw, _run
    # (the planner call describes 16-bit K/V; over 8-bit pages up to 32 query
    # vectors per KV head take the narrow kernel)
    assert rows * hq // hkv <= 32
    print(f"case narrow q8 {name}: H={history} R={rows} {hq}/{hkv} d={d} ps={ps} {dtype}", flush=True)
    case = synth.make_q8_case(name, history, rows, hq, hkv, d, ps, dtype, seed=history + rows + d)
    dev = _dev_q8(case)
    out = _run(dev, case, n_splits=n_splits)
    torch.cuda.synchronize()
    got = _gpu.host_out(out)
    if dtype == "f16":
        _gpu.assert_close(got, _oracle(case), name)
    else:
        _gpu.assert_close_bf16_bound(got, _oracle(case), _oracle_absw(case), name)


# Every build of the narrow kernel: head dimension x element type x 16 or 32
# query vectors per wave (rows x group at most 16 takes the 16 x 16 MFMAs;
# 17-32 exist for 8-bit pages, the 16-bit calls run the prefill kernel),
# a ragged context over several splits.
BUILDS = [(d, dt, nq) for d in (64, 128, 256) for dt in ("f16", "bf16") for nq in (16, 32)]


@pytest.mark.parametrize("d,dtype,nq", BUILDS, ids=[f"d{d}-{dt}-nq{nq}" for d, dt, nq in BUILDS])
def test_narrow_every_build(d, dtype, nq):
    import torch
    from test_gpu_q8 import _dev_q8, _oracle, _oracle_absw, _run
    rows, hq, hkv = (1, 16, 2) if nq == 16 else (2, 32, 2)   # 8 or 32 query vectors per KV head
    history = 2345 + d
    plan = pkg.paged_prefill_plan(history, rows, hq, hkv, d, 16, 0)
    assert (plan["m_tile"] == 32) == (nq == 16), plan
    print(f"case narrow build d={d} {dtype} nq={nq}: S={plan['n_splits']}", flush=True)
    case = synth.make_case("build", history, rows, hq, hkv, d, 16, dtype, seed=d + nq)
    dev = _gpu.dev_case(case, contiguous=False)
    out = pkg.paged_prefill_attention(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], history)
    torch.cuda.synchronize()
    _check(case, out, f"16-bit d={d} {dtype} nq={nq}")
    qc = synth.make_q8_case("build_q8", history, rows, hq, hkv, d, 16, dtype, seed=d + nq + 1)
    out8 = _run(_dev_q8(qc), qc)
    torch.cuda.synchronize()
    got = _gpu.host_out(out8)
    if dtype == "f16":
        _gpu.assert_close(got, _oracle(qc), f"q8 d={d} nq={nq}")
    else:
        _gpu.assert_close_bf16_bound(got, _oracle(qc), _oracle_absw(qc), f"q8 d={d} nq={nq}")


def test_narrow_repeat_calls_are_bitwise_identical():
    """The narrow kernel and its merge use no atomics and combine waves and
    splits in a fixed order: the same call gives the same bits every time,
    over 16-bit and 8-bit pages, with the workgroups' waves finishing in any
    order."""
    import torch
    from test_gpu_q8 import _dev_q8, _run
    case = synth.make_case("narrow_det", 20000, 1, 32, 4, 128, 16, "bf16", seed=12)
    dev = _gpu.dev_case(case, contiguous=False)
    outs = [pkg.paged_prefill_attention(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], case.history)
            for _ in range(4)]
    qc = synth.make_q8_case("narrow_det_q8", 20000, 2, 32, 2, 256, 16, "f16", seed=13)
    dq = _dev_q8(qc)
    outs8 = [_run(dq, qc) for _ in range(4)]
    torch.cuda.synchronize()
    assert all(_gpu.bits_equal(o, outs[0]) for o in outs[1:])
    assert all(_gpu.bits_equal(o, outs8[0]) for o in outs8[1:])
