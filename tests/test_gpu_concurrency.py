"""Calls from two host threads on two streams at once (the header's thread
safety: the split workspace is per (device, stream)).  Each thread runs a
sequence of calls whose workspace needs grow and shrink, so workspaces are
reallocated while the other thread's work is queued; every output must equal,
bit for bit, the same call made alone (the kernels are deterministic for a
given plan)."""

import threading

import pytest

import _gpu
import paged_kv_prefill_amd as pkg
from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

# (name, history, rows, Hq, Hkv, d, page size, dtype, splits): the split
# counts make the workspace grow within each thread's sequence
SEQ_A = [("a0", 3000, 64, 16, 2, 256, 16, "f16", 2), ("a1", 3000, 64, 16, 2, 256, 16, "f16", 8),
         ("a2", 1500, 200, 16, 2, 256, 16, "f16", 16), ("a3", 3000, 64, 16, 2, 256, 16, "f16", 3)]
SEQ_B = [("b0", 5000, 100, 32, 4, 128, 32, "bf16", 4), ("b1", 800, 300, 32, 4, 128, 32, "bf16", 12),
         ("b2", 5000, 100, 32, 4, 128, 32, "bf16", 1), ("b3", 5000, 100, 32, 4, 128, 32, "bf16", 24)]


def _cases(seq, seed):
    out = []
    for i, (name, h, r, hq, hkv, d, ps, dt, s) in enumerate(seq):
        case = synth.make_case(name, h, r, hq, hkv, d, ps, dt, seed=seed + i)
        out.append((case, _gpu.dev_case(case, contiguous=False), s))
    return out


def _call(case, dev, s, stream):
    return pkg.paged_prefill_attention(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"], case.history,
                                       n_splits=s, stream=stream)


def test_two_threads_on_two_streams():
    import torch
    print("case concurrency: two threads, two streams, 4 shapes x 6 rounds each", flush=True)
    ca, cb = _cases(SEQ_A, 100), _cases(SEQ_B, 200)
    # references: each call alone on the default stream
    ref_a = [_call(c, d, s, None) for c, d, s in ca]
    ref_b = [_call(c, d, s, None) for c, d, s in cb]
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    start = threading.Barrier(2)
    results = {"a": [], "b": []}
    errors = []

    def worker(key, cases, stream):
        try:
            start.wait()
            with torch.cuda.stream(stream):
                for _ in range(6):
                    for c, d, s in cases:
                        results[key].append(_call(c, d, s, stream))
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    ta = threading.Thread(target=worker, args=("a", ca, sa))
    tb = threading.Thread(target=worker, args=("b", cb, sb))
    ta.start()
    tb.start()
    ta.join()
    tb.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for key, refs in (("a", ref_a), ("b", ref_b)):
        got = results[key]
        assert len(got) == 6 * len(refs)
        for j, out in enumerate(got):
            assert _gpu.bits_equal(out, refs[j % len(refs)]), f"thread {key} call {j}"


def test_two_threads_on_one_stream():
    """Two host threads calling on the same stream at once: a call holds the
    stream's workspace until its merge kernel is enqueued, so one call's
    partials are never overwritten by the other thread's attention kernel
    before its merge reads them, also while the workspace grows."""
    import torch
    print("case concurrency: two threads, one stream, 4 shapes x 6 rounds each", flush=True)
    ca, cb = _cases(SEQ_A, 300), _cases(SEQ_B, 400)
    ref_a = [_call(c, d, s, None) for c, d, s in ca]
    ref_b = [_call(c, d, s, None) for c, d, s in cb]
    torch.cuda.synchronize()
    shared = torch.cuda.Stream()                 # default priority
    start = threading.Barrier(2)
    results = {"a": [], "b": []}
    errors = []

    def worker(key, cases):
        try:
            start.wait()
            with torch.cuda.stream(shared):
                for _ in range(6):
                    for c, d, s in cases:
                        results[key].append(_call(c, d, s, shared))
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    ta = threading.Thread(target=worker, args=("a", ca))
    tb = threading.Thread(target=worker, args=("b", cb))
    ta.start()
    tb.start()
    ta.join()
    tb.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for key, refs in (("a", ref_a), ("b", ref_b)):
        got = results[key]
        assert len(got) == 6 * len(refs)
        for j, out in enumerate(got):
            assert _gpu.bits_equal(out, refs[j % len(refs)]), f"thread {key} call {j}"
