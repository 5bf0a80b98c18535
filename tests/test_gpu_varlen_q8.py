"""GPU parity of multi-sequence (varlen) attention over 8-bit pages, through
the C ABI: packed batches of sequences with their own histories, rows and
block tables over one pool of quants and scales, against the fp64 oracle of
the dequantized pool (attention over 8-bit pages is the attention of the
dequantized K/V; a batch gives each sequence the single-sequence result).
Batches of decode steps run the narrow kernel (16 and 32 query vectors per
KV head); the others the prefill kernel widening each tile (one and two
query blocks per wave).  A one-sequence decode batch gives the bits of the
single call."""

import numpy as np
import pytest

import _gpu
import oracle
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

BATCHES = [
    # name, seqs [(history, rows)], Hq, Hkv, d, ps, shared [(dst, src, pages)]
    ("decode_nq16_d128", [(h, 1) for h in (0, 17, 300, 1023, 2500, 4999, 64, 777)], 16, 2, 128, 16, []),
    ("decode_nq32_d256", [(3000, 2), (45, 2), (1200, 1), (0, 2), (2047, 2)], 32, 2, 256, 32, []),
    ("decode_shared_d64", [(900, 1), (900, 1), (1500, 2), (0, 0)], 8, 1, 64, 16, [(1, 0, 56)]),
    ("prefill_d128", [(0, 37), (1000, 1), (333, 100), (64, 0), (2047, 65)], 8, 2, 128, 16, [(2, 4, 4)]),
    ("prefill_d64_two_blocks", [(500, 70), (10, 130), (2000, 40)], 8, 2, 64, 64, []),
    ("prefill_d256_ps256", [(700, 40), (130, 2), (0, 90)], 16, 2, 256, 256, [(1, 0, 1)]),
]


def _dev(case):
    import torch
    dev = "cuda:0"
    return {"q": _gpu.to_dev(case.q, _gpu.torch_dtype(case.dtype)),
            "kq": torch.from_numpy(case.k_quant).to(dev), "ks": torch.from_numpy(case.k_scale.view(np.int16)).to(dev),
            "vq": torch.from_numpy(case.v_quant).to(dev), "vs": torch.from_numpy(case.v_scale.view(np.int16)).to(dev),
            "bt": torch.from_numpy(case.block_tables).to(dev), "cu": torch.from_numpy(case.cu_rows).to(dev),
            "hist": torch.from_numpy(case.history_lens).to(dev)}


def _run(d, case, n_splits=0):
    return pkg.paged_prefill_attention_varlen_q8(d["q"], d["kq"], d["ks"], d["vq"], d["vs"], d["bt"], d["cu"],
                                                 d["hist"], case.max_rows, case.max_context, n_splits=n_splits)


def _oracle(case, abs_v=False):
    dec = oracle.decode_f16 if case.dtype == "f16" else oracle.decode_bf16
    k = oracle.dequantize_q8(case.k_quant, oracle.decode_scales(case.k_scale))
    v = oracle.dequantize_q8(case.v_quant, oracle.decode_scales(case.v_scale))
    return oracle.varlen_paged_attention(dec(case.q), k, np.abs(v) if abs_v else v, case.block_tables,
                                         case.cu_rows, case.history_lens, case.page_size)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("name,seqs,hq,hkv,d,ps,shared", BATCHES, ids=[b[0] for b in BATCHES])
def test_varlen_q8_matches_oracle(name, seqs, hq, hkv, d, ps, shared, dtype):
    import torch
    case = synth.make_varlen_q8_case(name, seqs, hq, hkv, d, ps, dtype, seed=len(seqs) + d, shared=shared)
    ref = _oracle(case)
    absw = _oracle(case, abs_v=True) if dtype == "bf16" else None
    dev = _dev(case)
    for s in (0, 1, 5):
        print(f"case varlen q8 {name} {dtype} S={s} (max rows {case.max_rows}, max context {case.max_context})",
              flush=True)
        out = _run(dev, case, n_splits=s)
        torch.cuda.synchronize()
        got = _gpu.host_out(out)
        if dtype == "f16":
            _gpu.assert_close(got, ref, f"{name} S={s}")
        else:
            _gpu.assert_close_bf16_bound(got, ref, absw, f"{name} S={s}")


@pytest.mark.parametrize("rows,hq,d", [(1, 16, 128), (2, 32, 256)])
def test_one_sequence_decode_batch_is_the_single_call(rows, hq, d):
    """A batch of one decode step has the single call's plan and kernel (the
    narrow kernel over 8-bit pages), so the same bits."""
    import torch
    history = 5000
    case = synth.make_varlen_q8_case("one_seq", [(history, rows)], hq, 2, d, 16, "bf16", seed=d + rows)
    dev = _dev(case)
    print(f"case varlen q8 one sequence R={rows} Hq={hq} d={d}", flush=True)
    got = _run(dev, case)
    single = pkg.paged_prefill_attention_q8(dev["q"], dev["kq"], dev["ks"], dev["vq"], dev["vs"], dev["bt"][0],
                                            history)
    torch.cuda.synchronize()
    assert _gpu.bits_equal(got, single)
