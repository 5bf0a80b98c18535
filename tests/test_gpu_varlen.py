"""GPU parity of multi-sequence (varlen) paged prefill, through the C ABI:
packed batches of sequences with their own histories, rows and block
tables over one pool (empty sequences, first chunks, single decode rows,
shared prefixes), against the fp64 oracle; and bit-for-bit equality with
one call per sequence under the same single-split plan."""

import numpy as np
import pytest

import _gpu
import oracle
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

BATCHES = [
    # name, seqs [(history, rows)], Hq, Hkv, d, ps, shared [(dst, src, pages)]
    ("mixed_d128", [(0, 37), (1000, 1), (333, 200), (5000, 16), (64, 0), (2047, 129)], 8, 2, 128, 16,
     [(3, 2, 10)]),
    ("mixed_d256", [(3000, 64), (0, 128), (17, 5), (1500, 1), (1500, 1)], 16, 2, 256, 16, [(4, 3, 93)]),
    ("ps8_d64", [(100, 50), (7, 3), (900, 20)], 4, 1, 64, 8, []),
    ("ps1_d128", [(50, 3), (0, 5), (9, 9)], 4, 2, 128, 1, [(2, 0, 9)]),
    ("ps128_d128", [(700, 40), (130, 2), (0, 300)], 12, 4, 128, 128, [(1, 0, 1)]),
    ("ps32_d256_mha", [(90, 7), (400, 33)], 2, 2, 256, 32, []),
]


def _dev(case):
    import torch
    dt = _gpu.torch_dtype(case.dtype)
    return {"q": _gpu.to_dev(case.q, dt), "kp": _gpu.to_dev(case.k_pages, dt), "vp": _gpu.to_dev(case.v_pages, dt),
            "bt": torch.from_numpy(case.block_tables).to("cuda:0"),
            "cu": torch.from_numpy(case.cu_rows).to("cuda:0"),
            "hist": torch.from_numpy(case.history_lens).to("cuda:0")}


def _run(d, case, n_splits=0):
    return pkg.paged_prefill_attention_varlen(d["q"], d["kp"], d["vp"], d["bt"], d["cu"], d["hist"], case.max_rows,
                                              case.max_context, n_splits=n_splits)


def _oracle(case):
    dec = oracle.decode_f16 if case.dtype == "f16" else oracle.decode_bf16
    return oracle.varlen_paged_attention(dec(case.q), dec(case.k_pages), dec(case.v_pages), case.block_tables,
                                         case.cu_rows, case.history_lens, case.page_size)


def _check(got, ref, case, what):
    # rows of an empty batch slot do not exist; every row belongs to a sequence here
    if case.dtype == "f16":
        _gpu.assert_close(got, ref, what)
    else:
        dec = oracle.decode_bf16
        absw = oracle.varlen_paged_attention(dec(case.q), dec(case.k_pages), np.abs(dec(case.v_pages)),
                                             case.block_tables, case.cu_rows, case.history_lens, case.page_size)
        _gpu.assert_close_bf16_bound(got, ref, absw, what)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name,seqs,hq,hkv,dim,ps,shared", BATCHES, ids=[b[0] for b in BATCHES])
def test_varlen_matches_oracle(name, seqs, hq, hkv, dim, ps, shared, dtype):
    import torch
    case = synth.make_varlen_case(name, seqs, hq, hkv, dim, ps, dtype, seed=len(seqs) * 11 + dim, shared=shared)
    plan = pkg.paged_prefill_plan_varlen(len(seqs), int(case.cu_rows[-1]), case.max_rows, case.max_context,
                                         hq, hkv, dim, ps)
    print(f"case varlen {name} {dtype}: {len(seqs)} seqs, {case.cu_rows[-1]} rows, planner S={plan['n_splits']} "
          f"grid={plan['grid']}", flush=True)
    d = _dev(case)
    ref = _oracle(case)
    for s in (0, 3):
        out = _run(d, case, n_splits=s)
        torch.cuda.synchronize()
        _check(_gpu.host_out(out), ref, case, f"{name} {dtype} S={s}")


@pytest.mark.parametrize("name,seqs,hq,hkv,dim,ps,shared", BATCHES[:2], ids=[b[0] for b in BATCHES[:2]])
def test_varlen_equals_one_call_per_sequence(name, seqs, hq, hkv, dim, ps, shared):
    """With one split every sequence's rows are computed by the same tile loop
    as a single-sequence call: the outputs agree bit for bit.  A single call
    of at most 32 query vectors per KV head runs the narrow kernel instead
    (its own summation order): those are held to the oracle."""
    import torch
    case = synth.make_varlen_case(name, seqs, hq, hkv, dim, ps, "bf16", seed=5, shared=shared)
    d = _dev(case)
    out = _run(d, case, n_splits=1)
    ref = absw = None
    n_bitwise = 0
    for s, (h, r) in enumerate(seqs):
        if r == 0:
            continue
        r0, r1 = int(case.cu_rows[s]), int(case.cu_rows[s + 1])
        one = pkg.paged_prefill_attention(d["q"][r0:r1].contiguous(), d["kp"], d["vp"], d["bt"][s].contiguous(), h,
                                          n_splits=1)
        torch.cuda.synchronize()
        if pkg.paged_prefill_plan(h, r, hq, hkv, dim, ps, 1)["m_tile"] == 32:
            if ref is None:
                dec = oracle.decode_bf16
                ref = _oracle(case)
                absw = oracle.varlen_paged_attention(dec(case.q), dec(case.k_pages), np.abs(dec(case.v_pages)),
                                                     case.block_tables, case.cu_rows, case.history_lens,
                                                     case.page_size)
            _gpu.assert_close_bf16_bound(_gpu.host_out(one), ref[r0:r1], absw[r0:r1], f"sequence {s} (narrow)")
        else:
            assert _gpu.bits_equal(one, out[r0:r1]), f"sequence {s}"
            n_bitwise += 1
    assert n_bitwise >= 2


def test_varlen_decode_batch():
    """32 sequences of one row each (a batch of decode steps) at histories
    from 1K to 32K, the planner's splits, all rows against the oracle."""
    import torch
    rng = np.random.default_rng(3)
    seqs = [(int(h), 1) for h in rng.integers(1024, 32768, size=32)]
    case = synth.make_varlen_case("decode32", seqs, 16, 2, 256, 16, "bf16", seed=12)
    plan = pkg.paged_prefill_plan_varlen(32, 32, 1, case.max_context, 16, 2, 256)
    print(f"case varlen decode batch: 32 x 1 row, H 1K-32K, S={plan['n_splits']}", flush=True)
    d = _dev(case)
    out = _run(d, case)
    torch.cuda.synchronize()
    got, ref = _gpu.host_out(out), _oracle(case)
    # Each sequence's rows are its own attention output: the stated tolerance
    # (with its rms floor) applies per sequence.  Over the whole batch the
    # floor would come from the short histories, whose outputs are larger.
    worst = 0.0
    for s in range(32):
        mabs, rel = _gpu.errors(got[s:s + 1], ref[s:s + 1])
        assert mabs <= _gpu.MAX_ABS and rel <= _gpu.MAX_REL, (s, seqs[s], mabs, rel)
        worst = max(worst, rel)
    print(f"  decode batch: worst per-sequence max_rel={worst:.3e}", flush=True)


# Batches of decode steps and short appends on the narrow kernel (every
# sequence at most 16 query vectors per KV head): empty sequences, first
# chunks (no history), histories shorter than a split (their later splits
# exit), pages of 8 and 64 tokens, one and 8-16 heads per KV head, split
# requests.
NARROW_BATCHES = [
    # name, seqs, Hq, Hkv, d, ps, dtype, n_splits
    ("nq16_d256", [(0, 1), (5000, 1), (37, 2), (64, 0), (20000, 2), (31, 1), (300, 1)], 16, 2, 256, 16, "bf16", 0),
    ("nq16_d128", [(4000, 2), (0, 1), (1234, 2), (9000, 1), (15, 2)], 16, 2, 128, 16, "f16", 0),
    ("g1_d64_ps8", [(700, 16), (3000, 5), (0, 0), (33, 9)], 1, 1, 64, 8, "f16", 0),
    ("nq16_d128_ps64_S3", [(6000, 2), (100, 1), (2500, 2)], 32, 4, 128, 64, "bf16", 3),
]


@pytest.mark.parametrize("name,seqs,hq,hkv,dim,ps,dtype,n_splits", NARROW_BATCHES, ids=[b[0] for b in NARROW_BATCHES])
def test_varlen_narrow_batches(name, seqs, hq, hkv, dim, ps, dtype, n_splits):
    import torch
    case = synth.make_varlen_case(name, seqs, hq, hkv, dim, ps, dtype, seed=len(seqs) + dim)
    plan = pkg.paged_prefill_plan_varlen(len(seqs), int(case.cu_rows[-1]), case.max_rows, case.max_context,
                                         hq, hkv, dim, ps, n_splits)
    assert plan["m_tile"] == 32, plan
    print(f"case varlen narrow {name}: {len(seqs)} seqs, max rows {case.max_rows}, S={plan['n_splits']} "
          f"grid={plan['grid']}", flush=True)
    d = _dev(case)
    out = _run(d, case, n_splits=n_splits)
    torch.cuda.synchronize()
    got, ref = _gpu.host_out(out), _oracle(case)
    # per sequence, as in the decode batch above
    for s, (h, r) in enumerate(seqs):
        if r == 0:
            continue
        r0, r1 = int(case.cu_rows[s]), int(case.cu_rows[s + 1])
        if dtype == "f16":
            _gpu.assert_close(got[r0:r1], ref[r0:r1], f"{name} sequence {s}")
        else:
            dec = oracle.decode_bf16
            absw = oracle.varlen_paged_attention(dec(case.q), dec(case.k_pages), np.abs(dec(case.v_pages)),
                                                 case.block_tables, case.cu_rows, case.history_lens, case.page_size)
            _gpu.assert_close_bf16_bound(got[r0:r1], ref[r0:r1], absw[r0:r1], f"{name} sequence {s}")


def test_varlen_prefill_batch_sampled():
    """Eight 256-row chunks at histories 8K-16K (d 256, fp16) in one launch;
    sampled rows against the oracle."""
    import torch
    seqs = [(8192 + 1024 * i, 256) for i in range(8)]
    case = synth.make_varlen_case("prefill8", seqs, 16, 2, 256, 16, "f16", seed=13)
    print("case varlen prefill batch: 8 x 256 rows, H 8K-15K", flush=True)
    d = _dev(case)
    out = _run(d, case)
    torch.cuda.synchronize()
    got = _gpu.host_out(out)
    dec = oracle.decode_f16
    picks = [0, 255, 256, 700, 1023, 1024, 1500, 2047]
    for s in range(8):
        rows = [p - 256 * s for p in picks if 256 * s <= p < 256 * (s + 1)]
        if not rows:
            continue
        k = oracle.gather_pages(dec(case.k_pages), case.block_tables[s], seqs[s][0] + 256, 16)
        v = oracle.gather_pages(dec(case.v_pages), case.block_tables[s], seqs[s][0] + 256, 16)
        ref = oracle.causal_attention_rows(dec(case.q[256 * s:256 * (s + 1)]), k, v, seqs[s][0], rows)
        _gpu.assert_close(got[[256 * s + r for r in rows]], ref, f"sequence {s} rows {rows}")


def test_varlen_empty_batches_are_no_ops():
    import torch
    case = synth.make_varlen_case("empty", [(10, 0), (0, 0)], 4, 1, 64, 16, "f16", seed=1)
    d = _dev(case)
    out = torch.empty((0, 4, 64), dtype=torch.float16, device="cuda:0")
    pkg.paged_prefill_attention_varlen(d["q"], d["kp"], d["vp"], d["bt"], d["cu"], d["hist"], 0, 10, out=out)
    torch.cuda.synchronize()
