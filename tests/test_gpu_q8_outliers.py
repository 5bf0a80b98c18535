"""Score outliers over 8-bit pages, through the C ABI against the fp64 oracle.
Every 8-bit path weighs scores in fp16 whatever the type of q (its MFMAs
take fp16 operands), so a key that scores about 16 log2 units or more above
a wave's reference overflows the weights and makes the wave raise its
reference and rescale O and l, in bf16 calls too.  One key per case (two
for "two_late") gets a first 32-value block of (127, 0, ..., 0) under a
large scale, and every query's component 0 is shifted by +2, so that key
scores about 2 * 127 * scale / sqrt(d) log2(e) above the rest for most rows.
The four paths: the narrow kernel with 16 and with 32 query vectors per KV
head, the prefill kernel widening tiles in its loop (fewer than four m tiles
per KV head), and the dequantize-once path (four or more), whose 16-bit
kernels run fp16 weights under a bf16 q as well.  Each runs at the
planner's split count and at one split (every wave then streams many
tiles, so a late outlier lands after its first).

The kernels' operands are the dequantized values rounded once to fp16.  The
planted scales are powers of two, so the planted values (127 * 2^k) are
exact in fp16 and the comparison with the exact oracle tests the softmax
alone.  With other scales an outlier component near 300 carries an fp16
rounding of up to 0.125, which moves its score by up to
|q_0| 0.125 / sqrt(d) log2(e) log2 units (a few percent of weight): two
outliers that share the weight then move the result by that share of
|V_1 - V_2|, whatever the arithmetic after the rounding (1e-2 with V rows of
unit size).  The last test keeps such scales and holds the kernels to the
stated tolerance against the oracle evaluated on the fp16-rounded
dequantized K/V."""

import numpy as np
import pytest

import _gpu
import oracle
from paged_kv_prefill_amd import synth
from test_gpu_q8 import _dev_q8, _oracle, _oracle_absw, _run

pytestmark = pytest.mark.gpu

PATHS = {
    # name: history, rows, Hq, Hkv, d (pages of 16 tokens)
    "narrow_nq16": (3000, 1, 16, 2, 128),     # 8 query vectors per KV head
    "narrow_nq32": (3000, 2, 32, 2, 256),     # 32
    "in_tile": (3000, 48, 8, 2, 128),         # 192: one 256-vector m tile per KV head
    "dequant_once": (1500, 256, 8, 2, 128),   # 1024: four m tiles per KV head
}

# (where, margin): the wanted margin of the outlier over the rest, in log2
# units, for a query whose shifted component 0 is 2; the scale is the power
# of two nearest to it (d 128: 8.1, 32.4, 64.8; d 256: 11.5, 22.9, 91.6).
# About 10 stays inside fp16's weights, the others overflow them.
OUTLIERS = [("late", 24.0), ("late", 76.0), ("first_tile", 76.0), ("two_late", 76.0), ("late", 10.0)]
LOG2E = float(np.log2(np.e))


def _outlier_scale(margin, d, exact):
    """Scale whose outlier value 127 * scale gives about `margin` log2 units;
    a power of two when `exact` (127 * 2^k is an fp16 value)."""
    s = margin * np.sqrt(d) / (2.0 * LOG2E) / 127.0
    if exact:
        s = 2.0 ** np.round(np.log2(s))
    return np.float16(s)


def _plant(case, keys_scales):
    """Shift q[., ., 0] by +2 and give each key its outlier block; its V row
    takes the scale 2^-8 (values quant / 256, exact in fp16, |V| < 0.5), so
    the rows it dominates have outputs well inside fp16's finest steps."""
    from paged_kv_prefill_amd.synth import ENCODERS
    dec = oracle.decode_f16 if case.dtype == "f16" else oracle.decode_bf16
    q = dec(case.q).astype(np.float32)
    q[:, :, 0] += 2.0
    case.q = ENCODERS[case.dtype](q)
    ps = case.page_size
    for key, scale in keys_scales:
        page, slot = case.block_table[key // ps], key % ps
        case.k_quant[page, slot, :, :32] = 0
        case.k_quant[page, slot, :, 0] = 127
        case.k_scale[page, slot, :, 0] = np.float16(scale).view(np.uint16)
        case.v_scale[page, slot] = np.float16(2.0 ** -8).view(np.uint16)
    return case


def _case(path, where, margin, dtype, exact):
    history, rows, hq, hkv, d = PATHS[path]
    case = synth.make_q8_case(f"q8_outlier_{path}", history, rows, hq, hkv, d, 16, dtype, seed=77 + rows)
    late = history - 100
    s = _outlier_scale(margin, d, exact)
    keys = {"late": [(late, s)], "first_tile": [(5, s)], "two_late": [(history // 2, s), (late, s)]}[where]
    return _plant(case, keys)


def _check_all_splits(case, ref, absw, what):
    import torch
    dev = _dev_q8(case)
    for s in (0, 1):
        print(f"case q8 outlier {what} {case.dtype} S={s}", flush=True)
        out = _run(dev, case, n_splits=s)
        torch.cuda.synchronize()
        got = _gpu.host_out(out)
        assert np.all(np.isfinite(got)), f"{what} S={s}: non-finite output"
        if case.dtype == "f16":
            _gpu.assert_close(got, ref, f"{what} S={s}")
        else:
            _gpu.assert_close_bf16_bound(got, ref, absw, f"{what} S={s}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("where,margin", OUTLIERS, ids=[f"{w}-{int(m)}" for w, m in OUTLIERS])
@pytest.mark.parametrize("path", list(PATHS))
def test_q8_score_outliers(path, where, margin, dtype):
    case = _case(path, where, margin, dtype, exact=True)
    absw = _oracle_absw(case) if dtype == "bf16" else None
    _check_all_splits(case, _oracle(case), absw, f"{path} {where} {margin}")


def _oracle_fp16_operands(case):
    """The oracle on K/V whose dequantized values are rounded to fp16 (the
    kernels' operand precision); q decoded exactly."""
    dec = oracle.decode_f16 if case.dtype == "f16" else oracle.decode_bf16
    ks, vs = oracle.decode_scales(case.k_scale), oracle.decode_scales(case.v_scale)
    ctx = case.history + case.rows
    kv = []
    for quant, sc in ((case.k_quant, ks), (case.v_quant, vs)):
        x = oracle.dequantize_q8(oracle.gather_pages(quant, case.block_table, ctx, case.page_size),
                                 oracle.gather_pages(sc, case.block_table, ctx, case.page_size))
        kv.append(x.astype(np.float16).astype(np.float64))
    return oracle.causal_attention(dec(case.q), kv[0], kv[1], case.history), kv


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("path", list(PATHS))
def test_q8_two_outliers_fp16_operands(path, dtype):
    """Two outliers under scales that are not powers of two (values near 300
    rounded to fp16 in the kernels): within the stated tolerance of the
    oracle on the fp16-rounded dequantized K/V."""
    case = _case(path, "two_late", 76.0, dtype, exact=False)
    ref, (k16, v16) = _oracle_fp16_operands(case)
    absw = None
    if dtype == "bf16":
        absw = oracle.causal_attention(oracle.decode_bf16(case.q), k16, np.abs(v16), case.history)
    _check_all_splits(case, ref, absw, f"{path} two_late fp16 operands")
