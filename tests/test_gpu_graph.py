"""The C ABI under HIP graph capture: once a stream's split workspace exists
(a first call on that stream), a call enqueues kernels only, so a serving loop
can capture it.  The captured piece loop (partial kernels and merges) is
replayed several times with new query values copied into the captured input
between replays and eager work of the program in between; every replay must
equal, bit for bit, the eager call on the same values.  A captured batch of
decode steps is also replayed as a serving loop would: with every sequence's
history grown in the device array between replays."""

import numpy as np
import pytest

import _gpu
import oracle
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


def test_replay_after_the_stream_workspace_grew():
    """A graph captured with a split call keeps working after later, larger
    calls on the same stream have grown its workspace (the smaller buffer is
    retired, not freed): each replay equals the eager call bit for bit."""
    import torch
    case = synth.make_case("graph_grow", 2048, 128, 16, 2, 256, 16, "f16", seed=33)
    big = synth.make_case("graph_big", 4096, 512, 16, 2, 256, 16, "f16", seed=34)
    print("case graph_grow: H=2048 R=128 16/2 d256 f16 S=4 captured; H=4096 R=512 S=8 between replays",
          flush=True)
    d = _gpu.dev_case(case, contiguous=False)
    db = _gpu.dev_case(big, contiguous=False)
    s = torch.cuda.Stream()                      # default priority
    out = torch.empty_like(d["q"])
    out_big = torch.empty_like(db["q"])

    def call(stream):
        pkg.paged_prefill_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], case.history,
                                    n_splits=4, out=out, stream=stream)

    def call_big(stream, splits):
        pkg.paged_prefill_attention(db["q"], db["k_pages"], db["v_pages"], db["block_table"], big.history,
                                    n_splits=splits, out=out_big, stream=stream)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
    torch.cuda.synchronize()
    eager = pkg.paged_prefill_attention(d["q"], d["k_pages"], d["v_pages"], d["block_table"], case.history,
                                        n_splits=4)
    torch.cuda.synchronize()
    before = pkg.paged_prefill_workspace_bytes(stream=s)
    for rep, splits in enumerate((8, 16)):
        with torch.cuda.stream(s):
            call_big(s, splits)                  # grows the capture stream's workspace
        s.synchronize()
        grown = pkg.paged_prefill_workspace_bytes(stream=s)
        assert grown > before, (before, grown)
        before = grown
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _gpu.bits_equal(out, eager), f"replay after growth {rep}"
        print(f"  replay after growth to {grown} bytes: equal to the eager call", flush=True)


def test_captured_decode_steps_replay():
    """Decode steps (the narrow kernel and the merge): one row over a paged
    history, and a batch of one-row sequences, captured once and replayed with
    new query values; every replay equals the eager call bit for bit."""
    import torch
    case = synth.make_case("graph_decode", 20000, 1, 16, 2, 256, 16, "bf16", seed=33)
    seqs = [(3000, 1), (0, 1), (12000, 1), (700, 0), (5000, 1)]
    vcase = synth.make_varlen_case("graph_decode_batch", seqs, 16, 2, 256, 16, "bf16", seed=34)
    assert pkg.paged_prefill_plan(case.history, 1, 16, 2, 256)["m_tile"] == 32
    print("case graph decode: H=20000 R=1 16/2 d256 bf16; batch of 5 sequences", flush=True)
    d = _gpu.dev_case(case, contiguous=False)
    dt = _gpu.torch_dtype(case.dtype)
    vq = _gpu.to_dev(vcase.q, dt)
    vk, vv = _gpu.to_dev(vcase.k_pages, dt), _gpu.to_dev(vcase.v_pages, dt)
    vbt = torch.from_numpy(vcase.block_tables).to("cuda:0")
    vcu = torch.from_numpy(vcase.cu_rows).to("cuda:0")
    vh = torch.from_numpy(vcase.history_lens).to("cuda:0")
    s = torch.cuda.Stream()
    q_in, vq_in = d["q"].clone(), vq.clone()
    out, vout = torch.empty_like(q_in), torch.empty_like(vq_in)

    def call(stream):
        pkg.paged_prefill_attention(q_in, d["k_pages"], d["v_pages"], d["block_table"], case.history, out=out,
                                    stream=stream)
        pkg.paged_prefill_attention_varlen(vq_in, vk, vv, vbt, vcu, vh, vcase.max_rows, vcase.max_context,
                                           out=vout, stream=stream)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    for rep in range(4):
        q_in.copy_(_gpu.to_dev(synth.ENCODERS["bf16"](rng.standard_normal(case.q.shape).astype(np.float32)), dt))
        vq_in.copy_(_gpu.to_dev(synth.ENCODERS["bf16"](rng.standard_normal(vcase.q.shape).astype(np.float32)), dt))
        g.replay()
        torch.cuda.synchronize()
        got, vgot = out.clone(), vout.clone()
        _ = (q_in.float() * 2).sum()
        eager = pkg.paged_prefill_attention(q_in, d["k_pages"], d["v_pages"], d["block_table"], case.history)
        veager = pkg.paged_prefill_attention_varlen(vq_in, vk, vv, vbt, vcu, vh, vcase.max_rows, vcase.max_context)
        torch.cuda.synchronize()
        assert _gpu.bits_equal(got, eager), f"replay {rep}"
        assert _gpu.bits_equal(vgot, veager), f"batch replay {rep}"
        print(f"  replay {rep}: equal to the eager calls", flush=True)


@pytest.mark.parametrize("q8", [False, True], ids=["16bit", "8bit"])
def test_captured_decode_batch_replays_with_growing_histories(q8):
    """A serving loop's decode step: a batch of one-row sequences captured
    once, with max_context a bound that leaves room to grow; between replays
    every sequence's history grows by one token (written into the device
    array in place) and the queries change.  The replays read the arrays as
    they are then: each equals the eager call on the same arrays bit for
    bit, and the oracle on the current histories."""
    import torch
    from test_gpu_varlen import _oracle as oracle16
    from test_gpu_varlen_q8 import _oracle as oracle8
    steps = 4
    start = [3000, 0, 12000, 700, 5000, 31]
    # the pools hold every token the steps reach: contexts start + steps + 1
    seqs = [(h + steps, 1) for h in start]
    dtype = "bf16"
    if q8:
        case = synth.make_varlen_q8_case("graph_grow_q8", seqs, 16, 2, 128, 16, dtype, seed=35)
    else:
        case = synth.make_varlen_case("graph_grow", seqs, 16, 2, 128, 16, dtype, seed=35)
    dt = _gpu.torch_dtype(dtype)
    dev = "cuda:0"
    q_in = _gpu.to_dev(case.q, dt).clone()
    bt = torch.from_numpy(case.block_tables).to(dev)
    cu = torch.from_numpy(case.cu_rows).to(dev)
    hist = torch.tensor(start, dtype=torch.int64, device=dev)
    bound = case.max_context
    out = torch.empty_like(q_in)
    if q8:
        pools = [torch.from_numpy(case.k_quant).to(dev), torch.from_numpy(case.k_scale.view(np.int16)).to(dev),
                 torch.from_numpy(case.v_quant).to(dev), torch.from_numpy(case.v_scale.view(np.int16)).to(dev)]
        call = lambda stream, o: pkg.paged_prefill_attention_varlen_q8(q_in, *pools, bt, cu, hist, 1, bound, out=o,
                                                                       stream=stream)
    else:
        kp, vp = _gpu.to_dev(case.k_pages, dt), _gpu.to_dev(case.v_pages, dt)
        call = lambda stream, o: pkg.paged_prefill_attention_varlen(q_in, kp, vp, bt, cu, hist, 1, bound, out=o,
                                                                    stream=stream)
    print(f"case graph decode batch, growing histories, {'8-bit' if q8 else '16-bit'} pages", flush=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s, out)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    for step in range(steps):
        hist.add_(1)
        q_new = synth.ENCODERS[dtype](rng.standard_normal(case.q.shape).astype(np.float32))
        q_in.copy_(_gpu.to_dev(q_new, dt))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = call(None, None)
        torch.cuda.synchronize()
        assert _gpu.bits_equal(got, eager), f"step {step}"
        case.q = q_new
        case.history_lens = hist.cpu().numpy()
        ref = oracle8(case) if q8 else oracle16(case)
        absw = oracle8(case, abs_v=True) if q8 else None
        if not q8:
            dec = oracle.decode_bf16
            absw = oracle.varlen_paged_attention(dec(case.q), dec(case.k_pages), np.abs(dec(case.v_pages)),
                                                 case.block_tables, case.cu_rows, case.history_lens, case.page_size)
        _gpu.assert_close_bf16_bound(_gpu.host_out(got), ref, absw, f"step {step}")
        print(f"  step {step}: histories {case.history_lens.tolist()}, equal to the eager call and within bound",
              flush=True)
