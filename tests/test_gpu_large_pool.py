"""Pools past 4 GiB, through the C ABI: the page addresses of the attention
loads (every addressing class), of the 8-bit pages and of both appends are
64-bit.  The pages a case uses sit at byte offsets between 2 and 5 GiB of
their pool (the last one past 4 GiB); every other slot of the pool holds NaN
(16-bit pools) or NaN scales (8-bit pools), so a wrong page poisons the
result.  The expected values come from the oracle on the same logical
tokens."""

import numpy as np
import pytest

import _gpu
import oracle
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

GIB = 1 << 30


def _high_table(rng, n_pages, page_bytes):
    """n_pages distinct pool pages at byte offsets in [2 GiB, 5 GiB), the last
    logical page in the pool's last page (past 4 GiB); returns (table, pool)."""
    lo, pool = (2 * GIB) // page_bytes, (5 * GIB) // page_bytes
    bt = (lo + rng.choice(pool - lo - 1, size=n_pages, replace=False)).astype(np.int32)
    bt[-1] = pool - 1
    assert int(bt.max()) * page_bytes >= 4 * GIB
    return bt, pool


def _fill_pool(pool_t, logical_pages, bt):
    """pool_t[bt[j]] = logical_pages[j] on the device."""
    import torch
    idx = torch.from_numpy(bt.astype(np.int64)).cuda()
    pool_t[idx] = logical_pages


def _logical_pages(tokens, page_size, fill):
    """[ctx][...] tokens padded to whole pages: [n_pages][ps][...]."""
    ctx = tokens.shape[0]
    n_pages = -(-ctx // page_size)
    pad = np.full((n_pages * page_size - ctx,) + tokens.shape[1:], fill, dtype=tokens.dtype)
    return np.concatenate([tokens, pad]).reshape((n_pages, page_size) + tokens.shape[1:])


CASES = [
    # name, history, rows, Hq, Hkv, d, page size, dtype (addressing class by page size)
    ("page16_f16_d256", 1000, 77, 16, 2, 256, 16, "f16"),
    ("pagebig_bf16_d128", 3000, 40, 8, 2, 128, 64, "bf16"),
    ("page8_f16_d64", 500, 33, 4, 1, 64, 8, "f16"),
    ("pagelane_bf16_d128", 700, 20, 8, 2, 128, 4, "bf16"),
    # decode steps: one row, at most 16 query vectors per KV head (the narrow kernel)
    ("narrow_f16_d128", 9000, 1, 16, 2, 128, 16, "f16"),
    ("narrow_bf16_d256_ps8", 5000, 1, 8, 1, 256, 8, "bf16"),
]


@pytest.mark.parametrize("name,history,rows,hq,hkv,dim,ps,dtype", CASES, ids=[c[0] for c in CASES])
def test_attention_reads_pages_past_4gib(name, history, rows, hq, hkv, dim, ps, dtype):
    import torch
    plan = pkg.paged_prefill_plan(history, rows, hq, hkv, dim, ps, 0)
    assert (plan["m_tile"] == 32) == name.startswith("narrow"), plan   # 32-key tiles: the narrow kernel
    case = synth.make_case(name, history, rows, hq, hkv, dim, ps, dtype, seed=rows + dim, table="identity")
    page_bytes = ps * hkv * dim * 2
    bt, pool = _high_table(np.random.default_rng(dim), -(-(history + rows) // ps), page_bytes)
    print(f"case large pool {name}: pool {pool} pages ({pool * page_bytes / GIB:.2f} GiB), "
          f"highest page at {int(bt.max()) * page_bytes / GIB:.2f} GiB", flush=True)
    dt = _gpu.torch_dtype(dtype)
    pools = []
    for tok in (case.k_contig, case.v_contig):
        p = torch.full((pool, ps, hkv, dim), -1, dtype=torch.int16, device="cuda:0")  # 0xFFFF: NaN
        _fill_pool(p, torch.from_numpy(_logical_pages(tok.view(np.int16), ps, np.int16(-1))).cuda(), bt)
        pools.append(p.view(dt))
    q = _gpu.to_dev(case.q, dt)
    bt_t = torch.from_numpy(bt).cuda()
    ref = _gpu.oracle_out(case)
    for s in (0, 3):
        out = pkg.paged_prefill_attention(q, pools[0], pools[1], bt_t, history, n_splits=s)
        torch.cuda.synchronize()
        got = _gpu.host_out(out)
        if dtype == "f16":
            _gpu.assert_close(got, ref, f"{name} S={s}")
        else:
            _gpu.assert_close_bf16_bound(got, ref, _gpu.oracle_abs_weighted(case), f"{name} S={s}")
    del pools
    torch.cuda.empty_cache()


# 64 rows take the prefill kernel; one row (8 query vectors per KV head) and
# 2 rows x 16 heads (32 per KV head) take the narrow kernel
Q8_CASES = [(1500, 64, 16, 2, 256), (6000, 1, 16, 2, 256), (4000, 2, 32, 2, 128)]


@pytest.mark.parametrize("history,rows,hq,hkv,dim", Q8_CASES, ids=[f"R{c[1]}_d{c[4]}" for c in Q8_CASES])
def test_q8_attention_reads_pages_past_4gib(history, rows, hq, hkv, dim):
    import torch
    ps = 16
    case = synth.make_q8_case("q8_large_pool", history, rows, hq, hkv, dim, ps, "f16", seed=9 + rows)
    n_pages = len(case.block_table)
    bt, pool = _high_table(np.random.default_rng(3), n_pages, ps * hkv * dim)
    print(f"case large pool q8 H={history} R={rows} d={dim}: pool {pool} pages ({pool * ps * hkv * dim / GIB:.2f} GiB of quants)", flush=True)
    dev = []
    for qp, sp in ((case.k_quant, case.k_scale), (case.v_quant, case.v_scale)):
        pq = torch.zeros((pool, ps, hkv, dim), dtype=torch.int8, device="cuda:0")
        psc = torch.full((pool, ps, hkv, dim // 32), -1, dtype=torch.int16, device="cuda:0")  # NaN scales
        _fill_pool(pq, torch.from_numpy(qp[case.block_table]).cuda(), bt)
        _fill_pool(psc, torch.from_numpy(sp[case.block_table].view(np.int16)).cuda(), bt)
        dev += [pq, psc]
    q = _gpu.to_dev(case.q, torch.float16)
    out = pkg.paged_prefill_attention_q8(q, dev[0], dev[1], dev[2], dev[3], torch.from_numpy(bt).cuda(), history)
    torch.cuda.synchronize()
    ks, vs = oracle.decode_scales(case.k_scale), oracle.decode_scales(case.v_scale)
    ref = oracle.paged_q8_attention(oracle.decode_f16(case.q), case.k_quant, ks, case.v_quant, vs,
                                    case.block_table, history, ps)
    _gpu.assert_close(_gpu.host_out(out), ref, "q8 pool past 4 GiB")
    del dev
    torch.cuda.empty_cache()


def test_appends_write_pages_past_4gib():
    """The 16-bit and the quantizing append into pages past 4 GiB: the
    appended slots hold the rows (the oracle's quantizer for 8-bit pages),
    and the rest of the pool is untouched."""
    import torch
    history, rows, hkv, dim, ps = 2040, 100, 2, 128, 16
    rng = np.random.default_rng(17)
    n_pages = -(-(history + rows) // ps)
    # 16-bit
    bt, pool = _high_table(rng, n_pages, ps * hkv * dim * 2)
    print(f"case large pool append: 16-bit pool {pool} pages, 8-bit pool after it", flush=True)
    kp = torch.full((pool, ps, hkv, dim), -1, dtype=torch.int16, device="cuda:0")
    vp = torch.full((pool, ps, hkv, dim), -1, dtype=torch.int16, device="cuda:0")
    k_new = rng.integers(0, 1 << 16, size=(rows, hkv, dim), dtype=np.uint16)   # any bit patterns: copied as is
    v_new = rng.integers(0, 1 << 16, size=(rows, hkv, dim), dtype=np.uint16)
    bt_t = torch.from_numpy(bt).cuda()
    pkg.paged_kv_append(_gpu.to_dev(k_new, torch.float16), _gpu.to_dev(v_new, torch.float16),
                        kp.view(torch.float16), vp.view(torch.float16), bt_t, history)
    torch.cuda.synchronize()
    pos = history + np.arange(rows)
    pages = torch.from_numpy(bt[pos // ps].astype(np.int64)).cuda()
    slots = torch.from_numpy((pos % ps).astype(np.int64)).cuda()
    for t, new in ((kp, k_new), (vp, v_new)):
        assert np.array_equal(t[pages, slots].cpu().numpy().view(np.uint16), new)
        t[pages, slots] = -1
        assert bool((t == -1).all())
    del kp, vp
    torch.cuda.empty_cache()
    # 8-bit
    bt, pool = _high_table(rng, n_pages, ps * hkv * dim)
    kq = torch.zeros((pool, ps, hkv, dim), dtype=torch.int8, device="cuda:0")
    vq = torch.zeros((pool, ps, hkv, dim), dtype=torch.int8, device="cuda:0")
    ksc = torch.zeros((pool, ps, hkv, dim // 32), dtype=torch.int16, device="cuda:0")
    vsc = torch.zeros((pool, ps, hkv, dim // 32), dtype=torch.int16, device="cuda:0")
    kn = synth.ENCODERS["bf16"](rng.standard_normal((rows, hkv, dim)).astype(np.float32))
    vn = synth.ENCODERS["bf16"](rng.standard_normal((rows, hkv, dim)).astype(np.float32))
    pkg.paged_kv_append_q8(_gpu.to_dev(kn, torch.bfloat16), _gpu.to_dev(vn, torch.bfloat16), kq, ksc, vq, vsc,
                           torch.from_numpy(bt).cuda(), history)
    torch.cuda.synchronize()
    pages = torch.from_numpy(bt[pos // ps].astype(np.int64)).cuda()
    for tq, tsc, new in ((kq, ksc, kn), (vq, vsc, vn)):
        wq, ws = oracle.quantize_q8(oracle.decode_bf16(new))
        assert np.array_equal(tq[pages, slots].cpu().numpy(), wq)
        assert np.array_equal(tsc[pages, slots].cpu().numpy().view(np.uint16), ws.view(np.uint16))
        tq[pages, slots] = 0
        tsc[pages, slots] = 0
        assert not bool(tq.any()) and not bool(tsc.any())
