"""The entry point that allocates nothing (paged_prefill_attention_pieces_noalloc):
its split workspace is the library's fixed device array.  Through the C ABI
it must give the same bits as the allocating entry point
(paged_prefill_attention_pieces, same plan and kernels) on two calls in a
row, the second smaller, without touching the per-stream workspaces; a call
whose plan needs more than the array holds is rejected before any launch."""

import ctypes

import pytest

import _gpu
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

SCRATCH_BYTES = 64 << 20


def _call_noalloc(**kw):
    a = dict(q=16, kp=16, vp=16, bt=16, H=10, R=4, P=0, hq=4, hkv=2, d=64, ps=16, S=0, out=4096, dt=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return pkg.lib().paged_prefill_attention_pieces_noalloc(
        vp(a["q"]), vp(a["kp"]), vp(a["vp"]), vp(a["bt"]), a["H"], a["R"], a["P"], a["hq"], a["hkv"], a["d"],
        a["ps"], a["S"], vp(a["out"]), a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), -4), (dict(R=-1), -2), (dict(d=96), -3), (dict(q=0), -1), (dict(out=16 + 64), -9),
    # 32 splits of a 2048-row chunk, 16 heads, d 256: 1 GiB of partials > 64 MiB
    (dict(H=32768, R=2048, hq=16, hkv=2, d=256, S=32, out=1 << 40), -5),
])
def test_noalloc_argument_errors_return_before_any_device_work(kw, code):
    assert _call_noalloc(**kw) == code


def test_noalloc_empty_chunk_is_a_no_op():
    assert _call_noalloc(R=0, q=0, kp=0, vp=0, bt=0, out=0) == 0


def test_planner_chunk_plans_fit_the_array():
    """The plans the workloads' pieces get fit the fixed array."""
    for h, r, hq, hkv, d in ((65536, 256, 32, 4, 128), (131072, 128, 16, 2, 256), (32768, 1, 16, 2, 256),
                             (8192, 512, 16, 2, 256)):
        assert pkg.paged_prefill_plan(h, r, hq, hkv, d)["workspace_bytes"] <= SCRATCH_BYTES


@pytest.mark.gpu
def test_noalloc_matches_the_allocating_entry_point_on_two_calls():
    import torch
    cases = [
        # (case, piece rows, split request)
        (synth.make_case("noalloc_a", 16384, 512, 32, 4, 128, 16, "bf16", seed=71), 256, 0),
        (synth.make_case("noalloc_b", 3000, 100, 16, 2, 256, 16, "f16", seed=72), 0, 5),
        # a decode step: the narrow kernel and the merge over the array
        (synth.make_case("noalloc_c", 20000, 1, 16, 2, 256, 16, "bf16", seed=73), 0, 0),
    ]
    s = torch.cuda.Stream()                      # default priority, no workspace yet
    for case, piece_rows, splits in cases:
        print(f"case {case.name}: H={case.history} R={case.rows} {case.n_q_heads}/{case.n_kv_heads} "
              f"d{case.head_dim} {case.dtype} pieces={piece_rows} S={splits}", flush=True)
        plan = pkg.paged_prefill_plan(case.history, piece_rows or case.rows, case.n_q_heads, case.n_kv_heads,
                                      case.head_dim, n_splits=splits)
        assert plan["n_splits"] > 1 and 0 < plan["workspace_bytes"] <= SCRATCH_BYTES
        d = _gpu.dev_case(case, contiguous=False)
        ref = pkg.paged_prefill_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], case.history,
                                          n_splits=splits, piece_rows=piece_rows)
        torch.cuda.synchronize()
        out = torch.full_like(d["q"], float("nan"))
        s.wait_stream(torch.cuda.current_stream())
        pkg.paged_prefill_attention_noalloc(d["q"], d["k_pages"], d["v_pages"], d["block_table"], case.history,
                                            n_splits=splits, out=out, piece_rows=piece_rows, stream=s)
        s.synchronize()
        assert _gpu.bits_equal(out, ref), case.name
        # the per-stream workspaces were not used
        assert pkg.paged_prefill_workspace_bytes(stream=s) == 0
        print("  bit-identical to paged_prefill_attention_pieces", flush=True)
