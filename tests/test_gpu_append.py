"""GPU parity of the KV append (paged_kv_append, through the C ABI) against
the oracle: the whole pool after the append, bit for bit."""

import numpy as np
import pytest

import oracle
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

POISON = 0xFFFF


def _pool_case(rng, history, rows, hkv, d, ps, extra_pool=5):
    """uint16 pools: history tokens random, every other slot POISON; a
    permuted block table; the chunk's rows to append."""
    ctx = history + rows
    n_pages = max(1, -(-ctx // ps))
    pool = n_pages + extra_pool
    bt = rng.permutation(pool)[:n_pages].astype(np.int32)
    kp = np.full((pool, ps, hkv, d), POISON, dtype=np.uint16)
    vp = np.full((pool, ps, hkv, d), POISON, dtype=np.uint16)
    for j in range(history):
        kp[bt[j // ps], j % ps] = rng.integers(0, 0x7C00, size=(hkv, d), dtype=np.uint16)
        vp[bt[j // ps], j % ps] = rng.integers(0, 0x7C00, size=(hkv, d), dtype=np.uint16)
    k_new = rng.integers(0, 1 << 16, size=(rows, hkv, d), dtype=np.uint16)
    v_new = rng.integers(0, 1 << 16, size=(rows, hkv, d), dtype=np.uint16)
    return kp, vp, bt, k_new, v_new


def _to_dev(a, dt):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).cuda()


def _to_host(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


SHAPES = [
    # history, rows, Hkv, d, ps
    (0, 1, 1, 64, 16), (0, 200, 2, 128, 16), (17, 5, 1, 64, 16), (1000, 77, 2, 128, 8),
    (333, 130, 2, 256, 16), (50, 3, 1, 128, 1), (700, 45, 2, 64, 32), (1500, 64, 1, 256, 256),
    (64, 64, 4, 64, 64), (5, 300, 3, 64, 4), (2047, 129, 2, 256, 1024),
]


@pytest.mark.parametrize("history,rows,hkv,d,ps", SHAPES, ids=[f"H{s[0]}-R{s[1]}-kv{s[2]}-d{s[3]}-ps{s[4]}" for s in SHAPES])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_append_matches_oracle(history, rows, hkv, d, ps, dtype):
    import torch
    import paged_kv_prefill_amd as pkg
    dt = torch.float16 if dtype == "f16" else torch.bfloat16
    rng = np.random.default_rng(history * 7 + rows)
    kp, vp, bt, k_new, v_new = _pool_case(rng, history, rows, hkv, d, ps)
    print(f"case append H={history} R={rows} Hkv={hkv} d={d} ps={ps} {dtype}", flush=True)
    dkp, dvp = _to_dev(kp, dt), _to_dev(vp, dt)
    pkg.paged_kv_append(_to_dev(k_new, dt), _to_dev(v_new, dt), dkp, dvp, torch.from_numpy(bt).cuda(), history)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.kv_append(kp, vp, bt, history, ps, k_new, v_new)
    assert np.array_equal(_to_host(dkp), ref_k)
    assert np.array_equal(_to_host(dvp), ref_v)


def test_append_then_attend_equals_contiguous():
    """Pages holding only the history (the chunk's slots poisoned), the chunk's
    K/V appended by the kernel, then the paged attention: bit-identical to the
    contiguous attention on the full K/V."""
    import torch
    import paged_kv_prefill_amd as pkg
    case = synth.make_case("append_attend", 1500, 300, 16, 2, 128, 16, "bf16", seed=31)
    dt = torch.bfloat16
    H, R, ps = case.history, case.rows, case.page_size
    kp, vp = case.k_pages.copy(), case.v_pages.copy()
    for i in range(R):
        pos = H + i
        kp[case.block_table[pos // ps], pos % ps] = POISON
        vp[case.block_table[pos // ps], pos % ps] = POISON
    q = _to_dev(case.q, dt)
    dkp, dvp = _to_dev(kp, dt), _to_dev(vp, dt)
    bt = torch.from_numpy(case.block_table).cuda()
    pkg.paged_kv_append(_to_dev(case.k_contig[H:], dt), _to_dev(case.v_contig[H:], dt), dkp, dvp, bt, H)
    out_p = pkg.paged_prefill_attention(q, dkp, dvp, bt, H)
    out_c = pkg.contiguous_prefill_attention(q, _to_dev(case.k_contig, dt), _to_dev(case.v_contig, dt), H)
    torch.cuda.synchronize()
    assert torch.equal(out_p.view(torch.int16), out_c.view(torch.int16))
    assert np.array_equal(_to_host(dkp), case.k_pages) and np.array_equal(_to_host(dvp), case.v_pages)


def test_append_full_chunk_in_a_large_pool():
    """A 2048-row chunk of the 128K workload's shape (16/2 heads, d 256) into
    a 65536-page pool through a scattered table: every appended row is checked
    against the chunk (oracle's placement rule, all 2048 rows), and nothing else
    in the pool changes (the pool with the chunk's slots masked is unchanged)."""
    import torch
    import paged_kv_prefill_amd as pkg
    H, R, hkv, d, ps, pool = 131072, 2048, 2, 256, 16, 65536
    rng = np.random.default_rng(41)
    n_pages = (H + R + ps - 1) // ps
    bt_np = rng.choice(pool, size=n_pages, replace=False).astype(np.int32)
    print(f"case append H={H} R={R} pool={pool} pages", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    kp = torch.randint(-32768, 32767, (pool, ps, hkv, d), dtype=torch.int16, device="cuda", generator=g)
    vp = torch.randint(-32768, 32767, (pool, ps, hkv, d), dtype=torch.int16, device="cuda", generator=g)
    k_new = rng.integers(0, 1 << 16, size=(R, hkv, d), dtype=np.uint16)
    v_new = rng.integers(0, 1 << 16, size=(R, hkv, d), dtype=np.uint16)
    kb, vb = kp.clone(), vp.clone()
    bt = torch.from_numpy(bt_np).cuda()
    pkg.paged_kv_append(_to_dev(k_new, torch.float16), _to_dev(v_new, torch.float16),
                        kp.view(torch.float16), vp.view(torch.float16), bt, H)
    torch.cuda.synchronize()
    pos = H + np.arange(R)
    pages = torch.from_numpy(bt_np[pos // ps].astype(np.int64)).cuda()
    slots = torch.from_numpy((pos % ps).astype(np.int64)).cuda()
    assert np.array_equal(kp[pages, slots].cpu().numpy().view(np.uint16), k_new)
    assert np.array_equal(vp[pages, slots].cpu().numpy().view(np.uint16), v_new)
    for t, b in ((kp, kb), (vp, vb)):
        t[pages, slots] = 0
        b[pages, slots] = 0
        assert torch.equal(t, b)
