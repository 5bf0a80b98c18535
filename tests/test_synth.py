"""The seeded input generators: rounding matches torch's own conversions,
the page layout matches the block table, unused slots hold the NaN poison."""

import numpy as np
import torch

from paged_kv_prefill_amd import synth


def test_encoders_round_to_nearest_even_like_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]  # exact ties
    ref_bf = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref_f16 = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.encode_bf16(x), ref_bf)
    assert np.array_equal(synth.encode_f16(x), ref_f16)


def test_layout_follows_block_table_and_poisons_the_rest():
    case = synth.make_case("t", 37, 6, 4, 2, 64, 16, "bf16", seed=5, table="scatter", pool_pages=50)
    ctx = case.ctx
    assert case.block_table.shape == (-(-ctx // 16),)
    assert len(set(case.block_table.tolist())) == len(case.block_table)
    for j in range(ctx):
        assert np.array_equal(case.k_pages[case.block_table[j // 16], j % 16], case.k_contig[j])
        assert np.array_equal(case.v_pages[case.block_table[j // 16], j % 16], case.v_contig[j])
    used = np.zeros(50, bool)
    used[case.block_table] = True
    assert np.all(case.k_pages[~used] == synth.POISON)
    assert np.all(case.v_pages[case.block_table[-1], ctx % 16:] == synth.POISON)


def test_seeded_cases_repeat():
    a = synth.config_case("tiny")
    b = synth.config_case("tiny")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_pages, b.k_pages)
    assert np.array_equal(a.block_table, b.block_table)
    assert sorted(a.block_table.tolist()) == list(range(36))


def test_exact_flops_counts_visible_keys():
    # 4 d Hq sum_i (H + i + 1) for R = 3, H = 5: (6 + 7 + 8) = 21
    assert synth.exact_flops(5, 3, 2, 8) == 4 * 8 * 2 * 21
