"""The C ABI under HIP graph capture: once a stream's split workspace exists
(a first call on that stream), a call enqueues kernels only, so a serving loop
can capture it.  The captured piece loop (partial kernels and merges) is
replayed several times with new query values copied into the captured input
between replays and eager work of the program in between; every replay must
equal, bit for bit, the eager call on the same values."""

import numpy as np
import pytest

import _gpu
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu


def test_captured_piece_loop_replays_match_eager_calls():
    import torch
    case = synth.make_case("graph", 4096, 256, 16, 2, 256, 16, "bf16", seed=31)
    print("case graph: H=4096 R=256 in 64-row pieces, 16/2 heads, d 256, bf16, 4 splits", flush=True)
    d = _gpu.dev_case(case, contiguous=False)
    dt = _gpu.torch_dtype(case.dtype)
    s = torch.cuda.Stream()                      # default priority
    q_in = d["q"].clone()
    out = torch.empty_like(q_in)

    def call(stream):
        pkg.paged_prefill_attention(q_in, d["k_pages"], d["v_pages"], d["block_table"], case.history,
                                    n_splits=4, out=out, piece_rows=64, stream=stream)

    # the first call on the capture stream sizes its workspace (hipMalloc), outside the capture
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for rep in range(4):
        q_new = synth.ENCODERS[case.dtype](rng.standard_normal(case.q.shape).astype(np.float32))
        q_in.copy_(_gpu.to_dev(q_new, dt))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        # eager work between replays, then the eager call on the same values
        _ = (q_in.float() * 2).sum()
        eager = pkg.paged_prefill_attention(q_in, d["k_pages"], d["v_pages"], d["block_table"], case.history,
                                            n_splits=4, piece_rows=64)
        torch.cuda.synchronize()
        assert _gpu.bits_equal(got, eager), f"replay {rep}"
        print(f"  replay {rep}: equal to the eager call", flush=True)
