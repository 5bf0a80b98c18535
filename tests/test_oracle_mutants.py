"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that at least one pin catches each of them: the pins are strong enough to
trust the oracle."""

import os
import types

import pytest

import _pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

ATTENTION_MUTANTS = [
    ("scale 1/d instead of 1/sqrt(d)",
     "    scale = 1.0 / math.sqrt(d)\n    out = np.empty", "    scale = 1.0 / d\n    out = np.empty"),
    ("exclusive causal diagonal",
     "visible = np.arange(n_keys)[None, :] <= last_visible[:, None]",
     "visible = np.arange(n_keys)[None, :] < last_visible[:, None]"),
    ("one key too many",
     "last_visible = history_len + np.repeat(rb, group)",
     "last_visible = history_len + 1 + np.repeat(rb, group)"),
    ("rows and heads of a group interleaved the wrong way",
     "last_visible = history_len + np.repeat(rb, group)",
     "last_visible = history_len + np.tile(rb, group)"),
    ("wrong KV head",
     "scores = (qb @ k[:n_keys, g, :].T) * scale",
     "scores = (qb @ k[:n_keys, (g + 1) % n_kv_heads, :].T) * scale"),
    ("K used in place of V",
     "(weights @ v[:n_keys, g, :])", "(weights @ k[:n_keys, g, :])"),
    ("normalised over the wrong axis",
     "weights = weights / weights.sum(axis=1, keepdims=True)",
     "weights = weights / weights.sum(axis=0, keepdims=True)"),
    ("block table ignored",
     "out[j] = pages[pool_page, j % page_size]", "out[j] = pages[j // page_size, j % page_size]"),
    ("page and slot swapped",
     "pool_page = block_table[j // page_size]", "pool_page = block_table[j % page_size]"),
    ("merge without the log-sum-exp normaliser",
     "weights = np.exp(lse - total[None])", "weights = np.exp(lse - top[None])"),
    ("wrong sign of ln l in lse",
     "m + np.log(safe_l)", "m - np.log(safe_l)"),
    ("exclusive diagonal in the split partials",
     "visible = np.arange(a, b)[None, :] <= last_visible[:, None]",
     "visible = np.arange(a, b)[None, :] < last_visible[:, None]"),
    ("split ranges drop their last key",
     "end = min((s + 1) * per * page_size, ctx)", "end = min((s + 1) * per * page_size - 1, ctx)"),
    ("partials not divided by their own sum",
     "o = (weights @ v[a:b, g, :]) / safe_l[:, None]", "o = (weights @ v[a:b, g, :])"),
    ("bfloat16 decoded with the wrong shift",
     "<< np.uint32(16)", "<< np.uint32(15)"),
    ("float16 decoded as bfloat16",
     "return np.asarray(raw, dtype=np.uint16).view(np.float16).astype(np.float64)",
     "return (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)"),
    ("row subset ignored",
     "rb = rows[b:b + block]\n", "rb = np.arange(len(rows))[b:b + block]\n"),
]

RULE_MUTANTS = [
    ("floor division replaced by the cap", "return min(max(per_head // tiles, 1), max_splits)",
     "return min(max(slot_cap // tiles, 1), max_splits)"),
    ("cores not divided by KV heads", "(per_core * gpu_cores) // kv_heads", "(per_core * gpu_cores)"),
    ("no clamp to max splits", "return min(max(per_head // tiles, 1), max_splits)",
     "return max(per_head // tiles, 1)"),
    ("piece budget off by a factor 2", "budget=1 << 25", "budget=1 << 26"),
    ("piece rule on history only", "rows * (history_len + rows) > budget", "rows * history_len > budget"),
]


CACHE_MUTANTS = [
    ("history ignored", "pos = history_len + i", "pos = i"),
    ("one position late", "pos = history_len + i", "pos = history_len + i + 1"),
    ("block table ignored", "pool_page = block_table[pos // page_size]", "pool_page = pos // page_size"),
    ("page and slot swapped", "pool_page = block_table[pos // page_size]", "pool_page = block_table[pos % page_size]"),
    ("slot from the page index", "slot = pos % page_size", "slot = (pos // page_size) % page_size"),
    ("V written into K", "k_out[pool_page, slot] = k_new[i]", "k_out[pool_page, slot] = v_new[i]"),
    ("input pool modified in place", "k_out = np.array(k_pages, copy=True)", "k_out = k_pages"),
    ("last row dropped", "for i in range(k_new.shape[0]):", "for i in range(k_new.shape[0] - 1):"),
]


VARLEN_MUTANTS = [
    ("first sequence's table for every sequence", "gather_pages(k_pages, block_tables[s], ctx, page_size)",
     "gather_pages(k_pages, block_tables[0], ctx, page_size)"),
    ("first sequence's history for every sequence", "hist = int(history_lens[s])", "hist = int(history_lens[0])"),
    ("row offset taken as the history", "hist = int(history_lens[s])", "hist = r0"),
    ("context without the chunk's own keys", "ctx = hist + (r1 - r0)", "ctx = hist"),
    ("last sequence dropped", "for s in range(len(history_lens)):", "for s in range(len(history_lens) - 1):"),
    ("last row of each sequence dropped", "r0, r1 = int(cu_rows[s]), int(cu_rows[s + 1])",
     "r0, r1 = int(cu_rows[s]), int(cu_rows[s + 1]) - 1"),
    ("rows taken from the start of q", "causal_attention(q[r0:r1], k, v, hist)",
     "causal_attention(q[:r1 - r0], k, v, hist)"),
    ("V gathered from the K pool", "v = gather_pages(v_pages, block_tables[s], ctx, page_size)",
     "v = gather_pages(k_pages, block_tables[s], ctx, page_size)"),
]


QUANT_MUTANTS = [
    ("scale over 128", "(amax / np.float32(127.0))", "(amax / np.float32(128.0))"),
    ("scale kept in fp32", "scale = (amax / np.float32(127.0)).astype(np.float16)",
     "scale = (amax / np.float32(127.0))"),
    ("scale from the signed max", "amax = np.abs(blocks).max(axis=-1)", "amax = blocks.max(axis=-1)"),
    ("ties rounded away from zero", "np.rint(blocks / safe)",
     "np.trunc(blocks / safe + np.copysign(np.float32(0.5), blocks))"),
    ("truncation instead of rounding", "np.rint(blocks / safe)", "np.trunc(blocks / safe)"),
    ("blocks of 16", "QBLOCK = 32", "QBLOCK = 16"),
    ("no clamp to 127", "q = np.clip(q, -127, 127).astype(np.int8)", "q = q.astype(np.int8)"),
    ("no saturation of the scale", "scale = np.minimum(scale, np.float16(FP16_MAX))", "scale = scale"),
    ("neighbouring block's scale", "s = np.asarray(scale).astype(np.float64)[..., None]",
     "s = np.roll(np.asarray(scale).astype(np.float64), 1, axis=-1)[..., None]"),
    ("V scales read from the K pool", "gather_pages(v_scale, block_table, ctx, page_size)",
     "gather_pages(k_scale, block_table, ctx, page_size)"),
    ("append one position late", "pos = history_len + i", "pos = history_len + i + 1"),
    ("append of V quantized from K", "vq, vs = quantize_q8(v_new)", "vq, vs = quantize_q8(k_new)"),
    ("scales decoded as bfloat16", "return np.asarray(raw, dtype=np.uint16).view(np.float16)",
     "return (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)"),
    ("scales decoded as integers", "return np.asarray(raw, dtype=np.uint16).view(np.float16)",
     "return np.asarray(raw, dtype=np.uint16).astype(np.float64)"),
    ("scale sign dropped", "return np.asarray(raw, dtype=np.uint16).view(np.float16)",
     "return np.abs(np.asarray(raw, dtype=np.uint16).view(np.float16))"),
]


def _mutated_module(filename, old, new):
    with open(os.path.join(ORACLE_DIR, filename)) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation target not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), filename, "exec"), mod.__dict__)
    return mod


def _caught(mod, pins):
    for pin in pins:
        try:
            pin(mod)
        except Exception:
            return True
    return False


@pytest.mark.parametrize("label,old,new", ATTENTION_MUTANTS, ids=[m[0] for m in ATTENTION_MUTANTS])
def test_attention_mutant_is_caught(label, old, new):
    mod = _mutated_module("attention.py", old, new)
    assert _caught(mod, _pins.ATTENTION_PINS), f"no pin caught: {label}"


@pytest.mark.parametrize("label,old,new", RULE_MUTANTS, ids=[m[0] for m in RULE_MUTANTS])
def test_rule_mutant_is_caught(label, old, new):
    mod = _mutated_module("rules.py", old, new)
    assert _caught(mod, _pins.RULE_PINS), f"no pin caught: {label}"


def test_unmutated_copy_passes_every_pin():
    mod = _mutated_module("attention.py", "import math", "import math")
    for pin in _pins.ATTENTION_PINS:
        pin(mod)


@pytest.mark.parametrize("label,old,new", CACHE_MUTANTS, ids=[m[0] for m in CACHE_MUTANTS])
def test_cache_mutant_is_caught(label, old, new):
    mod = _mutated_module("cache.py", old, new)
    assert _caught(mod, _pins.CACHE_PINS), f"no pin caught: {label}"


@pytest.mark.parametrize("label,old,new", VARLEN_MUTANTS, ids=[m[0] for m in VARLEN_MUTANTS])
def test_varlen_mutant_is_caught(label, old, new):
    mod = _mutated_module("varlen.py", old, new)
    assert _caught(mod, _pins.VARLEN_PINS), f"no pin caught: {label}"


@pytest.mark.parametrize("label,old,new", QUANT_MUTANTS, ids=[m[0] for m in QUANT_MUTANTS])
def test_quant_mutant_is_caught(label, old, new):
    mod = _mutated_module("quant.py", old, new)
    assert _caught(mod, _pins.QUANT_PINS), f"no pin caught: {label}"
