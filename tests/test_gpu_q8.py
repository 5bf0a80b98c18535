"""GPU parity of 8-bit KV pages, through the C ABI: the quantizing append
bit for bit against the oracle's quantizer, and the attention over 8-bit
pages (dequantized in the gather) against the fp64 oracle of the
dequantized K/V."""

import numpy as np
import pytest

import _gpu
import oracle
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu


def _dev_q8(case):
    import torch
    dev = "cuda:0"
    return {"q": _gpu.to_dev(case.q, _gpu.torch_dtype(case.dtype)),
            "kq": torch.from_numpy(case.k_quant).to(dev), "ks": torch.from_numpy(case.k_scale.view(np.int16)).to(dev),
            "vq": torch.from_numpy(case.v_quant).to(dev), "vs": torch.from_numpy(case.v_scale.view(np.int16)).to(dev),
            "bt": torch.from_numpy(case.block_table).to(dev)}


def _run(d, case, n_splits=0, piece_rows=0):
    return pkg.paged_prefill_attention_q8(d["q"], d["kq"], d["ks"], d["vq"], d["vs"], d["bt"], case.history,
                                          n_splits=n_splits, piece_rows=piece_rows)


def _oracle(case, rows=None):
    dec = oracle.decode_f16 if case.dtype == "f16" else oracle.decode_bf16
    ks, vs = oracle.decode_scales(case.k_scale), oracle.decode_scales(case.v_scale)
    if rows is None:
        return oracle.paged_q8_attention(dec(case.q), case.k_quant, ks, case.v_quant, vs, case.block_table,
                                         case.history, case.page_size)
    ctx = case.history + case.rows
    k = oracle.dequantize_q8(oracle.gather_pages(case.k_quant, case.block_table, ctx, case.page_size),
                             oracle.gather_pages(ks, case.block_table, ctx, case.page_size))
    v = oracle.dequantize_q8(oracle.gather_pages(case.v_quant, case.block_table, ctx, case.page_size),
                             oracle.gather_pages(vs, case.block_table, ctx, case.page_size))
    return oracle.causal_attention_rows(dec(case.q), k, v, case.history, np.asarray(rows))


def _oracle_absw(case):
    """sum_j p_j |V_j| for the bf16 bound."""
    dec = oracle.decode_bf16
    ks, vs = oracle.decode_scales(case.k_scale), oracle.decode_scales(case.v_scale)
    ctx = case.history + case.rows
    k = oracle.dequantize_q8(oracle.gather_pages(case.k_quant, case.block_table, ctx, case.page_size),
                             oracle.gather_pages(ks, case.block_table, ctx, case.page_size))
    v = oracle.dequantize_q8(oracle.gather_pages(case.v_quant, case.block_table, ctx, case.page_size),
                             oracle.gather_pages(vs, case.block_table, ctx, case.page_size))
    return oracle.causal_attention(dec(case.q), k, np.abs(v), case.history)


SHAPES = [
    # name, history, rows, Hq, Hkv, d, ps, n_splits
    ("first_chunk_d64", 0, 37, 4, 1, 64, 16, 0),
    ("ragged_d128", 1000, 77, 8, 2, 128, 16, 0),
    ("ragged_d256_S3", 333, 130, 16, 2, 256, 16, 3),
    ("ps32_d128", 700, 45, 8, 2, 128, 32, 2),
    ("ps64_d256", 1500, 64, 8, 1, 256, 64, 0),
    ("ps256_d64", 2100, 40, 12, 4, 64, 256, 2),
    ("one_row_long_d256", 4000, 1, 16, 2, 256, 16, 0),
    ("tail_d128", 2047, 129, 4, 2, 128, 16, 5),
    # four m tiles per KV head or more: the context is dequantized once into
    # fp16 and the 16-bit kernels run over it (the others widen in the tile loop)
    ("many_rows_d128", 500, 300, 8, 2, 128, 16, 0),
    ("many_rows_d64_S3", 200, 160, 16, 2, 64, 32, 3),
    ("many_rows_d256_ps64", 900, 70, 16, 2, 256, 64, 0),
]
CASES = [s[:7] + (dt,) + s[7:] for s in SHAPES for dt in ("f16", "bf16")]


@pytest.mark.parametrize("name,history,rows,hq,hkv,dim,ps,dtype,n_splits", CASES, ids=[f"{c[0]}-{c[7]}" for c in CASES])
def test_q8_attention_matches_oracle(name, history, rows, hq, hkv, dim, ps, dtype, n_splits):
    import torch
    case = synth.make_q8_case(name, history, rows, hq, hkv, dim, ps, dtype, seed=history + rows + dim)
    print(f"case q8 {name} {dtype}: H={history} R={rows} {hq}/{hkv} d={dim} ps={ps} S={n_splits}", flush=True)
    d = _dev_q8(case)
    out = _run(d, case, n_splits=n_splits)
    torch.cuda.synchronize()
    got = _gpu.host_out(out)
    ref = _oracle(case)
    if dtype == "f16":
        _gpu.assert_close(got, ref, name)
    else:
        _gpu.assert_close_bf16_bound(got, ref, _oracle_absw(case), name)


def _append_inputs(rng, rows, hkv, dim, dtype):
    """Random rows with planted blocks: all zero, the hand-quantized block,
    ties at +-k.5 steps, and (bf16) values past fp16's range."""
    import _pins
    x = rng.standard_normal((rows, hkv, dim)).astype(np.float32) * np.float32(0.7)
    x[0, 0, :32] = 0.0
    vals, _, _ = _pins.load_q8_golden()
    x[min(1, rows - 1), 0, 32:32 + len(vals)] = vals
    x[min(1, rows - 1), 0, 32 + len(vals):64] = 0.0
    if dtype == "bf16":
        x[-1, -1, :4] = [1.0e7, -3.0e6, 2.5e5, 1.0]
    enc = synth.ENCODERS[dtype]
    return enc(x)


APPEND = [(0, 5, 1, 64, 16), (17, 40, 2, 128, 16), (1000, 77, 2, 256, 32), (3, 130, 4, 64, 64), (500, 2048, 2, 256, 16)]


@pytest.mark.parametrize("history,rows,hkv,dim,ps", APPEND, ids=[f"H{a[0]}-R{a[1]}-d{a[3]}-ps{a[4]}" for a in APPEND])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_append_q8_matches_oracle_bit_for_bit(history, rows, hkv, dim, ps, dtype):
    import torch
    rng = np.random.default_rng(rows + dim)
    print(f"case append q8 H={history} R={rows} Hkv={hkv} d={dim} ps={ps} {dtype}", flush=True)
    ctx = history + rows
    n_pages = -(-ctx // ps)
    pool = n_pages + 3
    bt = rng.permutation(pool)[:n_pages].astype(np.int32)
    kq = rng.integers(-128, 128, size=(pool, ps, hkv, dim), dtype=np.int8)
    vq = rng.integers(-128, 128, size=(pool, ps, hkv, dim), dtype=np.int8)
    ks = rng.integers(0, 1 << 16, size=(pool, ps, hkv, dim // 32), dtype=np.uint16)
    vs = rng.integers(0, 1 << 16, size=(pool, ps, hkv, dim // 32), dtype=np.uint16)
    kn = _append_inputs(rng, rows, hkv, dim, dtype)
    vn = _append_inputs(rng, rows, hkv, dim, dtype)
    dev = "cuda:0"
    dt = _gpu.torch_dtype(dtype)
    t = [torch.from_numpy(a.copy()).to(dev) for a in (kq, ks.view(np.int16), vq, vs.view(np.int16))]
    pkg.paged_kv_append_q8(_gpu.to_dev(kn, dt), _gpu.to_dev(vn, dt), t[0], t[1], t[2], t[3],
                           torch.from_numpy(bt).to(dev), history)
    torch.cuda.synchronize()
    dec = oracle.decode_f16 if dtype == "f16" else oracle.decode_bf16
    want = oracle.kv_append_q8(kq, ks, vq, vs, bt, history, ps, dec(kn), dec(vn))
    got = [t[0].cpu().numpy(), t[1].cpu().numpy().view(np.uint16), t[2].cpu().numpy(), t[3].cpu().numpy().view(np.uint16)]
    for g, w, what in zip(got, want, ("k quants", "k scales", "v quants", "v scales")):
        assert np.array_equal(g, w), what


def test_q8_pieces_dequantized_once():
    """A bf16 chunk in 128-row pieces over 8-bit pages with 32/4 heads, d 128:
    the context is dequantized once for all pieces and every piece runs the
    two-block 16-bit kernel over it; all rows against the oracle."""
    import torch
    case = synth.make_q8_case("q8_pieces", 1000, 512, 32, 4, 128, 16, "bf16", seed=88, piece_rows=128)
    print("case q8 pieces: H=1000 R=512 in 128-row pieces, 32/4 heads, d 128, bf16", flush=True)
    d = _dev_q8(case)
    out = _run(d, case, piece_rows=128)
    torch.cuda.synchronize()
    _gpu.assert_close_bf16_bound(_gpu.host_out(out), _oracle(case), _oracle_absw(case), "q8 pieces")


@pytest.mark.parametrize("name", ["sweep_32768", "piece_64k", "long_128k"])
def test_q8_full_size_sampled(name):
    """The 32K chunk (fp16, one call), the 64K chunk (bf16, 8 pieces of 256
    rows, d 128) and the 128K chunk (bf16, 16 pieces of 128 rows, pages
    scattered over a 65,536-page pool) over 8-bit pages of the same shapes;
    sampled rows against the oracle."""
    import torch
    base = synth.config_case(name)
    case = synth.make_q8_case(name, base.history, base.rows, base.n_q_heads, base.n_kv_heads, base.head_dim,
                              base.page_size, base.dtype, seed=77, table="scatter" if name == "long_128k" else "permute",
                              pool_pages=65536 if name == "long_128k" else None, piece_rows=base.piece_rows)
    del base
    print(f"case q8 {name}: H={case.history} R={case.rows} pieces={case.piece_rows}", flush=True)
    d = _dev_q8(case)
    out = _run(d, case, piece_rows=case.piece_rows)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    rows = np.unique(np.r_[0, 1, case.rows - 1, case.rows // 2, np.random.default_rng(5).integers(0, case.rows, 12)])
    _gpu.assert_close(got[rows].astype(np.float64), _oracle(case, rows), f"{name} q8 on {len(rows)} rows")
