"""Oracle of quantized KV pages: 8-bit K/V dequantized in the gather.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy, one
block at a time in spirit (vectorised over blocks only), float64 for the
attention.  Shares no code with the HIP library.

The report "Research: KVarN V-store per-call latency grows with n_kv at
fixed grid, K stays flat" measures its KV formats against q8_0, the 8-bit
KV cache type of the engine it runs on (its throughput table), and the
speculative-decoding page runs its engine with an int8 KV cache (its
"Engine arguments").  Neither page spells the format out; the reading here
is q8_0's structure: each (token, KV head) row of d values is cut into
blocks of 32 consecutive values along d, and each block stores

  scale = the block's max |x| / 127, rounded to fp16 (saturated at 65504),
  q_i   = x_i / scale rounded to the nearest integer, ties to even,
          clamped to [-127, 127]  (0 for an all-zero block),

so that the block's values are read back as scale * q_i.  The division and
the scale are fp32 operations on the exact input values (fp16 and bf16 are
exact in fp32), then the scale is rounded once to fp16: both sides of a
test can reproduce every bit.  The quants and the scales live in two pools
with the page layout of the 16-bit cache:
  quants [n_pool_pages][ps][Hkv][d]      int8
  scales [n_pool_pages][ps][Hkv][d / 32] fp16 (bit patterns as uint16)
Attention over such pages is the attention of the dequantized K and V.
"""

import numpy as np

from oracle.attention import causal_attention, gather_pages

QBLOCK = 32
FP16_MAX = 65504.0


def quantize_q8(x):
    """(q int8 [..., d], scale fp16 [..., d/32]) of values x [..., d]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % QBLOCK == 0
    blocks = x.astype(np.float32).reshape(x.shape[:-1] + (d // QBLOCK, QBLOCK))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(over="ignore"):
        scale = (amax / np.float32(127.0)).astype(np.float16)
    scale = np.minimum(scale, np.float16(FP16_MAX))
    s = scale.astype(np.float32)[..., None]
    safe = np.where(s > 0, s, np.float32(1.0))
    q = np.where(s > 0, np.rint(blocks / safe), np.float32(0.0))
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(x.shape), scale


def dequantize_q8(q, scale):
    """float64 values scale * q, block by block (exact)."""
    q = np.asarray(q)
    d = q.shape[-1]
    blocks = q.astype(np.float64).reshape(q.shape[:-1] + (d // QBLOCK, QBLOCK))
    s = np.asarray(scale).astype(np.float64)[..., None]
    return (blocks * s).reshape(q.shape)


def decode_scales(raw):
    """fp16 bit patterns (uint16) -> float16 values."""
    return np.asarray(raw, dtype=np.uint16).view(np.float16)


def paged_q8_attention(q, k_quant, k_scale, v_quant, v_scale, block_table, history_len, page_size):
    """Causal attention of the chunk (rows at H .. H+R-1) over q8 pages:
    gather quants and scales through the block table, dequantize, then the
    same definition as for 16-bit pages.  q: float [R][Hq][d]; scales as
    float16 values (see decode_scales)."""
    ctx = history_len + np.asarray(q).shape[0]
    k = dequantize_q8(gather_pages(k_quant, block_table, ctx, page_size),
                      gather_pages(k_scale, block_table, ctx, page_size))
    v = dequantize_q8(gather_pages(v_quant, block_table, ctx, page_size),
                      gather_pages(v_scale, block_table, ctx, page_size))
    return causal_attention(q, k, v, history_len)


def kv_append_q8(k_quant, k_scale, v_quant, v_scale, block_table, history_len, page_size, k_new, v_new):
    """The q8 pools after quantizing k_new/v_new [R][Hkv][d] into positions
    H .. H+R-1 (slot (H+i) mod ps of page block_table[(H+i) div ps]).
    Returns new arrays; nothing else changes."""
    outs = [np.array(a, copy=True) for a in (k_quant, k_scale, v_quant, v_scale)]
    kq, ks = quantize_q8(k_new)
    vq, vs = quantize_q8(v_new)
    for i in range(np.asarray(k_new).shape[0]):
        pos = history_len + i
        page = block_table[pos // page_size]
        slot = pos % page_size
        outs[0][page, slot] = kq[i]
        outs[1][page, slot] = ks[i].view(outs[1].dtype) if outs[1].dtype == np.uint16 else ks[i]
        outs[2][page, slot] = vq[i]
        outs[3][page, slot] = vs[i].view(outs[3].dtype) if outs[3].dtype == np.uint16 else vs[i]
    return tuple(outs)
