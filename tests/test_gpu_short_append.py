"""Short appends and decode steps on a long history: R from 1 to 288 rows
after 32K-128K tokens (the issue's 922-token continuation and the PR's
278-288-row appends, scaled to the long workloads' histories), where the
planner cuts the history into up to 128 splits.  HIP path through the C ABI
against the fp64 oracle; paged against contiguous bit for bit."""

import numpy as np
import pytest

import _gpu
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

# name, history, Hq, Hkv, d, dtype, pool pages (None: a permutation of the pages used)
HISTORIES = [
    ("h32k_d256_f16", 32768, 16, 2, 256, "f16", None),
    ("h64k_d128_bf16", 65536, 32, 4, 128, "bf16", None),
    ("h128k_d256_bf16", 131072, 16, 2, 256, "bf16", 65536),
]
ROWS = (1, 3, 16, 100, 288)
MAX_ROWS = max(ROWS)


@pytest.fixture(scope="module", params=HISTORIES, ids=[h[0] for h in HISTORIES])
def long_case(request):
    import torch
    name, history, hq, hkv, d, dtype, pool = request.param
    print(f"case {name}: H={history} up to {MAX_ROWS} rows", flush=True)
    case = synth.make_case(name, history, MAX_ROWS, hq, hkv, d, 16, dtype, seed=17,
                           table="scatter" if pool else "permute", pool_pages=pool)
    dev = _gpu.dev_case(case)
    q = _gpu.decode(case, case.q)
    k = _gpu.decode(case, case.k_contig)
    v = _gpu.decode(case, case.v_contig)
    yield case, dev, (q, k, v)
    del dev
    torch.cuda.empty_cache()


def _oracle_rows(qkv, history, rows):
    import oracle
    q, k, v = qkv
    return oracle.causal_attention_rows(q, k, v, history, np.asarray(rows))


@pytest.mark.parametrize("rows", ROWS)
def test_short_append_matches_oracle(long_case, rows):
    import torch
    case, d, qkv = long_case
    H = case.history
    plan = pkg.paged_prefill_plan(H, rows, case.n_q_heads, case.n_kv_heads, case.head_dim, 16)
    print(f"case {case.name} R={rows}: planner splits {plan['n_splits']}, grid {plan['grid']}", flush=True)
    q = d["q"][:rows].contiguous()
    out = pkg.paged_prefill_attention(q, d["k_pages"], d["v_pages"], d["block_table"], H)
    out_c = pkg.contiguous_prefill_attention(q, d["k"], d["v"], H)
    torch.cuda.synchronize()
    assert _gpu.bits_equal(out, out_c), "paged and contiguous differ bitwise"
    picks = np.arange(rows) if rows <= 16 else np.unique(np.r_[0, 1, rows // 2, rows - 2, rows - 1,
                                                             np.random.default_rng(rows).integers(0, rows, 7)])
    ref = _oracle_rows(qkv, H, picks)
    _gpu.assert_close(_gpu.host_out(out)[picks], ref, f"{case.name} R={rows} S={plan['n_splits']} rows {len(picks)}")


@pytest.mark.parametrize("n_splits", [256, 100000])
def test_decode_step_with_many_splits(long_case, n_splits):
    """One row with the split count forced far past the planner's: 256, and
    one split per 64-key unit (the request is clamped to the unit count), so
    the merge combines up to ~2K partials per output."""
    import torch
    case, d, qkv = long_case
    H = case.history
    plan = pkg.paged_prefill_plan(H, 1, case.n_q_heads, case.n_kv_heads, case.head_dim, 16, n_splits)
    print(f"case {case.name} R=1 S={plan['n_splits']} (requested {n_splits})", flush=True)
    q = d["q"][:1].contiguous()
    out = pkg.paged_prefill_attention(q, d["k_pages"], d["v_pages"], d["block_table"], H, n_splits=n_splits)
    out_c = pkg.contiguous_prefill_attention(q, d["k"], d["v"], H, n_splits=n_splits)
    torch.cuda.synchronize()
    assert _gpu.bits_equal(out, out_c)
    _gpu.assert_close(_gpu.host_out(out)[[0]], _oracle_rows(qkv, H, [0]), f"{case.name} R=1 S={plan['n_splits']}")



def test_decode_and_append_on_a_4m_token_history():
    """A decode step and a 16-row append after 4,194,304 tokens (2^22; d 64,
    8/1 heads, fp16): key positions far past the long workloads', the
    planner's 128 splits; paged = contiguous bit for bit and every row
    against the oracle."""
    import torch
    H, R = 1 << 22, 16
    case = synth.make_case("h4m_d64_f16", H, R, 8, 1, 64, 16, "f16", seed=23)
    d = _gpu.dev_case(case)
    outs = []
    for rows in (1, R):
        plan = pkg.paged_prefill_plan(H, rows, 8, 1, 64, 16)
        print(f"case h4m R={rows}: planner splits {plan['n_splits']}", flush=True)
        q = d["q"][:rows].contiguous()
        out = pkg.paged_prefill_attention(q, d["k_pages"], d["v_pages"], d["block_table"], H)
        out_c = pkg.contiguous_prefill_attention(q, d["k"], d["v"], H)
        torch.cuda.synchronize()
        assert _gpu.bits_equal(out, out_c), f"R={rows}: paged and contiguous differ bitwise"
        outs.append(_gpu.host_out(out))
    del d
    torch.cuda.empty_cache()
    qkv = tuple(_gpu.decode(case, a) for a in (case.q, case.k_contig, case.v_contig))
    ref = _oracle_rows(qkv, H, np.arange(R))
    _gpu.assert_close(outs[0], ref[:1], "H=4M R=1")
    _gpu.assert_close(outs[1], ref, "H=4M R=16")
