"""Benchmark: paged prefill attention, TFLOP/s and ms per 2048-row chunk at
32K-128K history, on one MI355X.

One step is one 2048-row chunk at each of three histories, paged KV with the
pages in random order (the workloads of the PR's attention sweep and the
issue's long prefill):
  * 32K history, 16 Q / 2 KV heads, d 256, fp16, the chunk in one call;
  * 64K history, 32 Q / 4 KV heads, d 128, bf16, eight 256-row pieces;
  * 128K history, 16 Q / 2 KV heads, d 256, bf16, sixteen 128-row pieces,
    pages scattered over a 65,536-page pool.
Inputs are resident in HBM before the timed region.  The contiguous-KV path
runs on the same values right after each paged chunk (A/B), outside the
step's value, and so are the per-chunk medians with a cold cache (a 512 MB
scratch write before each call, more than the 256 MB Infinity Cache plus the
8 x 4 MB L2) in rounds alternating with warm calls.  Also outside it (skip
with --no-extra): the paged/contiguous ratio of the
2048-row chunk at 1K-16K history and of the Qwen-like chunk, split-count
sweeps on the 32K chunk and on the 64K and 128K pieces against the planner,
peaked-score inputs, the KV append of each chunk (GB/s against HBM peak), short appends
/ decode steps (1-288 rows) on each chunk's history, multi-sequence batches
in one launch against one call per sequence, and each chunk over 8-bit K/V
pages.  Prints one JSON line.

With --power SECONDS it also runs each chunk, and an 8192^3 fp16 matmul, back
to back for SECONDS while sampling board power and engine clocks.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-ab] [--no-extra] [--copy-calibration]
                  [--power SECONDS]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0
NOMINAL_CLOCK_GHZ = 2.4   # the engine clock the published peaks assume
CHUNKS = ("sweep_32768", "piece_64k", "long_128k")
ROOFLINE_CHUNK = "sweep_32768"   # one attention launch per call (one split, no merge)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-ab", action="store_true", help="skip the contiguous-KV A/B")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the cold-cache, short-history and split-count measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (known bytes) for counter scaling")
    ap.add_argument("--chunks", default=",".join(CHUNKS))
    ap.add_argument("--decode-only", action="store_true",
                    help="only a one-row decode step over each chunk's history (16-bit and 8-bit pages), "
                         "K timed calls each, printed as its own JSON line (a short run for counter passes)")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="also run each chunk (and an fp16 matmul) back to back for SECONDS each while "
                         "sampling board power and engine clocks with amd-smi")
    return ap.parse_args()


def kernel_source_hash():
    from paged_kv_prefill_amd.profsum import kernel_source_hash as h
    return h()


def load_traffic(kernel_hash):
    """HBM bytes per launch of the roofline kernel from the committed counter
    summary, or None if the kernel changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "attn_d256_f16_paged_32k_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def load_clock(kernel_hash):
    """The engine clock the roofline kernel ran at (an upper bound from the
    committed MFMA counter pass), or None if the kernel changed since."""
    path = os.path.join(ROOT, "profiles", "attn_d256_f16_paged_32k_mfma_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_hash:
        return None
    return rec.get("clock_ghz_upper_bound")


def load_power(kernel_hash):
    """Sustained board power, engine clock and rate of the roofline chunk and of
    an fp16 matmul under the same power limit, from the committed summary of a
    `--power` run, or None if the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "power_clock_sustained_chunks_and_f16_matmul.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_hash:
        return None
    return rec.get("phases")


def cpu_baseline(cases, budget_s=15.0):
    """The oracle (numpy float64) on a bounded sample of the step's chunks,
    timed on this host's cores: evenly spaced rows of each chunk in turn
    (the 32K chunk first), until about budget_s seconds of oracle work;
    reported in TFLOP/s of exact causal FLOPs."""
    import numpy as np
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:
        threads = os.cpu_count()
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu_model)
    except OSError:
        pass
    total_flops, total_s, parts = 0.0, 0.0, []
    for case in cases:
        left = budget_s - total_s
        if left < 1.0:
            break
        dec = oracle.decode_f16 if case.dtype == "f16" else oracle.decode_bf16
        q, k, v = dec(case.q), dec(case.k_contig), dec(case.v_contig)

        def flops(rows):
            return sum(4 * case.head_dim * case.n_q_heads * (case.history + int(r) + 1) for r in rows)

        probe = np.arange(0, case.rows, max(1, case.rows // 16))
        t0 = time.perf_counter()
        oracle.causal_attention_rows(q, k, v, case.history, probe)
        dt_probe = time.perf_counter() - t0
        per_row = dt_probe / len(probe)
        n = int(min(case.rows, max(16, left / max(per_row, 1e-6))))
        rows = np.unique(np.linspace(0, case.rows - 1, n).astype(np.int64))
        t0 = time.perf_counter()
        oracle.causal_attention_rows(q, k, v, case.history, rows)
        dt = time.perf_counter() - t0
        total_flops += flops(rows)
        total_s += dt
        parts.append(f"{len(rows)} of {case.rows} rows of the {case.history // 1024}K-history chunk")
        del q, k, v
    return {"value": total_flops / total_s / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": ", ".join(parts) + f" (rows evenly spaced), {total_s:.1f} s, numpy float64 with BLAS on "
                      f"{threads} threads",
            "seconds": total_s, "cpu_model": cpu_model, "blas": blas}


def power_measurements(chunks, paged, stream, seconds):
    """Board power and engine clock under sustained load: each chunk called back
    to back for `seconds`, and an 8192^3 fp16 matmul (torch, i.e. the vendor
    GEMM library) as the reference of what dense MFMA work reaches under the
    same board power limit.  A thread samples `amd-smi metric -p -c` (socket
    power, the eight XCDs' GFX clocks) every ~0.2 s; a phase reports the median
    power and the mean clock of the samples taken from 1 s after its start to
    its end, and its own rate."""
    import re
    import subprocess
    import threading
    import numpy as np
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            t = time.time()
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c"], capture_output=True, text=True,
                                   timeout=10)
                pw = re.search(r"SOCKET_POWER: (\d+) W", r.stdout)
                clk = [int(x) for x in re.findall(r"GFX_\d+:\s+CLK: (\d+) MHz", r.stdout)]
                if pw and clk:
                    samples.append((t, int(pw.group(1)), float(np.mean(clk))))
            except (OSError, subprocess.SubprocessError):
                return
            stop.wait(0.2)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    phases = {}

    def phase(name, fn, flops):
        fn()
        torch.cuda.synchronize()
        t0, n = time.time(), 0
        while time.time() - t0 < seconds:
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            n += 5
        t1 = time.time()
        phases[name] = (t0, t1, (t1 - t0) / n * 1e3, flops)
        print(f"# power phase {name}: {n} calls", file=sys.stderr, flush=True)

    time.sleep(2.0)
    phases["idle"] = (time.time() - 2.0, time.time(), None, None)
    n_g = 8192
    a = torch.randn(n_g, n_g, device=stream.device, dtype=torch.float16)
    b = torch.randn(n_g, n_g, device=stream.device, dtype=torch.float16)
    cg = torch.empty_like(a)
    phase("matmul_f16_8192", lambda: torch.matmul(a, b, out=cg), 2.0 * n_g ** 3)
    del a, b, cg
    for c in chunks:
        phase(c["name"], lambda: paged(c), c["flops"])
    stop.set()
    th.join(timeout=15)
    res = {"samples": len(samples)}
    for name, (t0, t1, ms, flops) in phases.items():
        sel = [x for x in samples if t0 + (0.0 if name == "idle" else 1.0) <= x[0] <= t1]
        rec = {"power_w_median": float(np.median([x[1] for x in sel])) if sel else None,
               "gfx_clock_mhz_mean": round(float(np.mean([x[2] for x in sel])), 1) if sel else None,
               "n_samples": len(sel)}
        if ms is not None:
            rec.update({"ms_per_call": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)})
        res[name] = rec
    return res


def stated_flops(case):
    """FLOPs in the convention 4 * rows * ctx * head_dim * n_q_heads with ctx =
    history + rows of each call (the chunk's pieces summed): counts the masked
    upper triangle of each call's own rows, 3% more than the exact count at
    32K, 0.8% at 128K."""
    p = case.piece_rows or case.rows
    total = 0
    for r0 in range(0, case.rows, p):
        r = min(p, case.rows - r0)
        total += 4 * r * (case.history + r0 + r) * case.head_dim * case.n_q_heads
    return total


def kv_bytes(case):
    """Algorithmic K+V bytes of one chunk: every key read once."""
    return (case.history + case.rows) * case.n_kv_heads * case.head_dim * 2 * 2


def timed(fn, reps, stream, before=None):
    """Median, p10, p90 ms of fn() over reps calls, each bracketed by events on
    `stream`; `before` (if given) runs before each call, outside the events."""
    import numpy as np
    import torch
    evs = []
    for _ in range(reps):
        if before is not None:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.median(ms)), float(np.percentile(ms, 10)), float(np.percentile(ms, 90))


def timed_cold_warm(fn, flush, rounds, reps, stream):
    """Median, p10, p90 ms of fn() with a cold cache (flush() before each
    call, outside its events) and warm (calls back to back), timed in
    alternating rounds of reps calls each, so that the chip's clock drift over
    the run reaches both alike.  Returns (cold, warm)."""
    import numpy as np
    import torch
    evs = {"cold": [], "warm": []}
    for _ in range(rounds):
        for kind in ("warm", "cold"):
            for _ in range(reps):
                if kind == "cold":
                    flush()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                evs[kind].append((a, b))
    torch.cuda.synchronize()
    stats = []
    for kind in ("cold", "warm"):
        ms = np.array([a.elapsed_time(b) for a, b in evs[kind]])
        stats.append((float(np.median(ms)), float(np.percentile(ms, 10)), float(np.percentile(ms, 90))))
    return stats[0], stats[1]


def timed_pair(fa, fb, reps, stream):
    """Medians of fa() and fb() called alternately (so clock drift hits both)."""
    import numpy as np
    import torch
    evs = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        fa()
        e[1].record(stream)
        e[2].record(stream)
        fb()
        e[3].record(stream)
        evs.append(e)
    torch.cuda.synchronize()
    return (float(np.median([e[0].elapsed_time(e[1]) for e in evs])),
            float(np.median([e[2].elapsed_time(e[3]) for e in evs])))


def timed_round_robin(fns, reps, stream, seed=5):
    """Median ms of each of several calls, timed in rounds (every call once
    per round, in a shuffled order) so that clock drift over the run, and the
    state a longer or shorter call leaves behind, hit all alike."""
    import numpy as np
    import torch
    for f in fns.values():
        f()
    evs = {k: [] for k in fns}
    rng = np.random.default_rng(seed)
    keys = list(fns)
    for _ in range(reps):
        for idx in rng.permutation(len(keys)):
            k, f = keys[idx], fns[keys[idx]]
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            b.record(stream)
            evs[k].append((a, b))
    torch.cuda.synchronize()
    return {k: round(float(np.median([a.elapsed_time(b) for a, b in v])), 4) for k, v in evs.items()}


def extra_measurements(chunks, paged, contig, pkg, synth, to_dev, stream, reps=10):
    """Cold-cache medians, the short-history sweep and the split sweep."""
    import torch
    out = {}
    sweep = {}
    for h in (1024, 2048, 4096, 8192, 16384):
        case = synth.config_case(f"sweep_{h}")
        dt = torch.float16 if case.dtype == "f16" else torch.bfloat16
        q, kp, vp = to_dev(case.q, dt), to_dev(case.k_pages, dt), to_dev(case.v_pages, dt)
        bt = torch.from_numpy(case.block_table).to(stream.device)
        k, v = to_dev(case.k_contig, dt), to_dev(case.v_contig, dt)
        o, oc = torch.empty_like(q), torch.empty_like(q)
        fp = lambda: pkg.paged_prefill_attention(q, kp, vp, bt, case.history, out=o, stream=stream)
        fc = lambda: pkg.contiguous_prefill_attention(q, k, v, case.history, out=oc, stream=stream)
        for _ in range(3):
            fp()
            fc()
        mp, mc = timed_pair(fp, fc, 2 * reps, stream)
        fl = synth.exact_flops(case.history, case.rows, case.n_q_heads, case.head_dim)
        sweep[f"{h // 1024}K"] = {"ms_median": round(mp, 4), "tflops": round(fl / (mp * 1e-3) / 1e12, 1),
                                  "contiguous_ms_median": round(mc, 4), "paged_over_contiguous": round(mp / mc, 4),
                                  "bitwise_equal_to_contiguous": bool(torch.equal(o.view(torch.int16),
                                                                                  oc.view(torch.int16)))}
        del q, kp, vp, bt, k, v, o, oc
    out["history_sweep_2048_rows"] = sweep
    # The Qwen-like chunk (8K history, 512 rows, values x 0.5), paged against contiguous.
    case = synth.config_case("qwen_like")
    q, kp, vp = to_dev(case.q, torch.float16), to_dev(case.k_pages, torch.float16), to_dev(case.v_pages, torch.float16)
    bt = torch.from_numpy(case.block_table).to(stream.device)
    k, v = to_dev(case.k_contig, torch.float16), to_dev(case.v_contig, torch.float16)
    o, oc = torch.empty_like(q), torch.empty_like(q)
    fp = lambda: pkg.paged_prefill_attention(q, kp, vp, bt, case.history, out=o, stream=stream)
    fc = lambda: pkg.contiguous_prefill_attention(q, k, v, case.history, out=oc, stream=stream)
    for _ in range(3):
        fp()
        fc()
    mp, mc = timed_pair(fp, fc, 2 * reps, stream)
    fl = synth.exact_flops(case.history, case.rows, case.n_q_heads, case.head_dim)
    out["qwen_like_8k_512_rows"] = {"ms_median": round(mp, 4), "tflops": round(fl / (mp * 1e-3) / 1e12, 1),
                                    "contiguous_ms_median": round(mc, 4), "paged_over_contiguous": round(mp / mc, 4),
                                    "splits": pkg.paged_prefill_plan(case.history, case.rows, 16, 2, 256)["n_splits"],
                                    "bitwise_equal_to_contiguous": bool(torch.equal(o.view(torch.int16),
                                                                                    oc.view(torch.int16)))}
    del q, kp, vp, bt, k, v, o, oc
    out["peaked_scores"] = peaked_measurements(chunks, paged, pkg, stream, reps)
    # Page-size sweep on the 32K chunk: the same K/V laid out in pages of 1 to
    # 256 tokens (a random page order), paged against contiguous, interleaved.
    c = next((c for c in chunks if c["name"] == "sweep_32768"), None)
    if c is not None:
        cs = c["case"]
        ctx = cs.history + cs.rows
        gen = torch.Generator(device="cpu").manual_seed(61)
        pss = {}
        for ps in (1, 4, 8, 16, 32, 64, 256):
            n_pages = ctx // ps
            perm = torch.randperm(n_pages, generator=gen).to(stream.device)
            kp = torch.empty((n_pages, ps, cs.n_kv_heads, cs.head_dim), dtype=c["k"].dtype, device=stream.device)
            vp = torch.empty_like(kp)
            kp[perm] = c["k"][:ctx].view(n_pages, ps, cs.n_kv_heads, cs.head_dim)
            vp[perm] = c["v"][:ctx].view(n_pages, ps, cs.n_kv_heads, cs.head_dim)
            bt = perm.to(torch.int32)
            o = torch.empty_like(c["q"])
            fp = lambda: pkg.paged_prefill_attention(c["q"], kp, vp, bt, cs.history, out=o, stream=stream)
            fc = lambda: contig(c)
            for _ in range(3):
                fp()
                fc()
            mp, mc = timed_pair(fp, fc, reps, stream)
            pss[str(ps)] = {"ms_median": round(mp, 4), "paged_over_contiguous": round(mp / mc, 4)}
            del kp, vp, bt, o, perm
        out["page_size_sweep_32k"] = pss
    # KV append of each chunk's own K/V rows into its pages (idempotent here):
    # bytes = K and V rows read once and written once
    app = {}
    for c in chunks:
        cs = c["case"]
        kn, vn = c["k"][cs.history:cs.history + cs.rows], c["v"][cs.history:cs.history + cs.rows]
        f = lambda: pkg.paged_kv_append(kn, vn, c["kp"], c["vp"], c["bt"], cs.history, stream=stream)
        for _ in range(3):
            f()
        ms = timed(f, 2 * reps, stream)[0]
        nbytes = 4 * cs.rows * cs.n_kv_heads * cs.head_dim * 2
        app[c["name"]] = {"ms_median": round(ms, 5), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bytes": nbytes}
    out["kv_append_2048_rows"] = app
    # steady state: the whole 32K history's K/V (positions 0 .. 32767) in one call
    c = next((c for c in chunks if c["name"] == "sweep_32768"), None)
    if c is not None:
        n = c["case"].history
        kn, vn = c["k"][:n], c["v"][:n]
        f = lambda: pkg.paged_kv_append(kn, vn, c["kp"], c["vp"], c["bt"], 0, stream=stream)
        f()
        ms = timed(f, 2 * reps, stream)[0]
        nbytes = 4 * n * c["case"].n_kv_heads * c["case"].head_dim * 2
        out["kv_append_32k_rows"] = {"ms_median": round(ms, 5), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                     "bytes": nbytes}
    c = next((c for c in chunks if c["name"] == "sweep_32768"), None)
    if c is not None:
        cs = c["case"]
        res = timed_round_robin(
            {str(sreq): (lambda sreq=sreq: pkg.paged_prefill_attention(c["q"], c["kp"], c["vp"], c["bt"], cs.history,
                                                                       n_splits=sreq, out=c["out"], stream=stream))
             for sreq in (1, 2, 4, 8, 16, 32)}, reps, stream)
        out["split_sweep_32k_ms_median"] = res
        out["split_sweep_planner_splits"] = pkg.paged_prefill_plan(cs.history, cs.rows, cs.n_q_heads,
                                                                   cs.n_kv_heads, cs.head_dim)["n_splits"]
    # The PR's comparison (1 split against the planner) at its piece shapes:
    # the whole 64K chunk in 256-row pieces and the 128K chunk in 128-row
    # pieces, every piece at the same requested split count; "planner" is each
    # piece's own planned count.
    for name, counts in (("piece_64k", (1, 2, 4, 8, 16, 32)), ("long_128k", (1, 4, 8, 16, 32, 64))):
        c = next((c for c in chunks if c["name"] == name), None)
        if c is None:
            continue
        cs = c["case"]
        res = timed_round_robin(
            {("planner" if sreq == 0 else str(sreq)):
             (lambda sreq=sreq: pkg.paged_prefill_attention(c["q"], c["kp"], c["vp"], c["bt"], cs.history,
                                                            n_splits=sreq, out=c["out"], piece_rows=cs.piece_rows,
                                                            stream=stream))
             for sreq in counts + (0,)}, reps, stream)
        best = min(v for k, v in res.items() if k != "planner")
        planned = pkg.paged_prefill_plan(cs.history, cs.piece_rows, cs.n_q_heads, cs.n_kv_heads,
                                         cs.head_dim)["n_splits"]
        out[f"split_sweep_{name}_ms_median"] = res
        out[f"split_sweep_{name}_planner_splits"] = planned
        # the planner's own count where the sweep has it (the same plan, timed in the same rounds)
        mine = res.get(str(planned), res["planner"])
        out[f"split_sweep_{name}_planner_over_best"] = round(mine / best, 4)
    # Short appends and decode steps: the first R rows of each chunk as one
    # call on the same history (planner splits).  KV-bound at small R, so
    # reported as K/V bytes per second against HBM peak, with the paged /
    # contiguous ratio (calls interleaved).
    short = {}
    for c in chunks:
        cs = c["case"]
        res = {}
        for r in (1, 16, 128, 288):
            q = c["q"][:r].contiguous()
            o, oc = torch.empty_like(q), torch.empty_like(q)
            fp = lambda: pkg.paged_prefill_attention(q, c["kp"], c["vp"], c["bt"], cs.history, out=o, stream=stream)
            fc = lambda: pkg.contiguous_prefill_attention(q, c["k"], c["v"], cs.history, out=oc, stream=stream)
            for _ in range(3):
                fp()
                fc()
            mp, mc = timed_pair(fp, fc, 2 * reps, stream)
            kvb = (cs.history + r) * cs.n_kv_heads * cs.head_dim * 2 * 2
            fl = synth.exact_flops(cs.history, r, cs.n_q_heads, cs.head_dim)
            res[f"R{r}"] = {"ms_median": round(mp, 5), "kv_gbs": round(kvb / (mp * 1e-3) / 1e9, 1),
                            "hbm_frac": round(kvb / (mp * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                            "tflops": round(fl / (mp * 1e-3) / 1e12, 1),
                            "splits": pkg.paged_prefill_plan(cs.history, r, cs.n_q_heads, cs.n_kv_heads,
                                                             cs.head_dim)["n_splits"],
                            "paged_over_contiguous": round(mp / mc, 4)}
        short[c["name"]] = res
    out["short_append_and_decode"] = short
    out["varlen"] = varlen_measurements(pkg, synth, stream, reps)
    out["q8_pages"] = q8_measurements(chunks, paged, pkg, synth, stream, reps)
    return out


def peaked_measurements(chunks, paged, pkg, stream, reps):
    """The 32K fp16 and 128K bf16 chunks with peaked scores: q scaled by 4
    (scores with sigma about 4 instead of 1) and component 0 of every query
    raised by 8, and eight keys spread over the last quarter of the history
    with component 0 set to 56, so that for most rows one late key scores
    12-20 nats (or more) above the split's first tile.  Where a weight would
    overflow, the wave raises its softmax reference and rescales its
    accumulators; the time is reported against the same chunk with N(0,1)
    inputs (calls interleaved)."""
    import torch
    res = {}
    for name in ("sweep_32768", "long_128k"):
        c = next((c for c in chunks if c["name"] == name), None)
        if c is None:
            continue
        cs = c["case"]
        q2 = (c["q"].float() * 4.0)
        q2[:, :, 0] += 8.0
        q2 = q2.to(c["q"].dtype)
        kp2 = c["kp"].clone()
        keys = [cs.history - 1 - (cs.history // 4) * j // 8 for j in range(8)]
        bt = c["bt"].cpu().numpy()
        for key in keys:
            kp2[int(bt[key // cs.page_size]), key % cs.page_size, :, 0] = 56.0
        o2 = torch.empty_like(c["q"])
        fpk = lambda: pkg.paged_prefill_attention(q2, kp2, c["vp"], c["bt"], cs.history, out=o2,
                                                  piece_rows=cs.piece_rows, stream=stream)
        fn = lambda: paged(c)
        for _ in range(3):
            fpk()
            fn()
        mp, mn = timed_pair(fpk, fn, reps, stream)
        res[name] = {"ms_median": round(mp, 4), "normal_inputs_ms_median": round(mn, 4),
                     "over_normal_inputs": round(mp / mn, 4),
                     "finite": bool(torch.isfinite(o2.float()).all())}
        del q2, kp2, o2
        torch.cuda.empty_cache()
    return res


def q8_pages_for(cs, synth, dev):
    """8-bit pages of the chunk case's shapes (random quants and scales; the
    128K chunk's pages scattered over a 65,536-page pool) on the device:
    (case, k quants, k scales, v quants, v scales, block table)."""
    import numpy as np
    import torch
    qc = synth.make_q8_case(cs.name, cs.history, cs.rows, cs.n_q_heads, cs.n_kv_heads, cs.head_dim, cs.page_size,
                            cs.dtype, seed=51, table="scatter" if cs.name == "long_128k" else "permute",
                            pool_pages=65536 if cs.name == "long_128k" else None, piece_rows=cs.piece_rows)
    return (qc, torch.from_numpy(qc.k_quant).to(dev), torch.from_numpy(qc.k_scale.view(np.int16)).to(dev),
            torch.from_numpy(qc.v_quant).to(dev), torch.from_numpy(qc.v_scale.view(np.int16)).to(dev),
            torch.from_numpy(qc.block_table).to(dev))


def decode_only(chunks, pkg, synth, stream, steps, warmup):
    """A one-row decode step (the chunk's first row) over each chunk's
    history: 16-bit pages, then 8-bit pages of the same shapes; median ms of
    `steps` calls after `warmup`, K/V bytes per second against HBM peak."""
    import torch
    res = {}
    for c in chunks:
        cs = c["case"]
        q1, o1 = c["q"][:1].contiguous(), torch.empty_like(c["q"][:1])
        f16 = lambda: pkg.paged_prefill_attention(q1, c["kp"], c["vp"], c["bt"], cs.history, out=o1, stream=stream)
        _, kq, ks, vq, vs, bt = q8_pages_for(cs, synth, stream.device)
        f8 = lambda: pkg.paged_prefill_attention_q8(q1, kq, ks, vq, vs, bt, cs.history, out=o1, stream=stream)
        rec = {}
        for name, f, row_bytes in (("16bit", f16, 2 * cs.head_dim), ("8bit", f8, cs.head_dim + cs.head_dim // 16)):
            for _ in range(warmup):
                f()
            ms = timed(f, steps, stream)[0]
            kvb = (cs.history + 1) * cs.n_kv_heads * row_bytes * 2
            rec[name] = {"ms_median": round(ms, 5), "kv_bytes": kvb, "kv_gbs": round(kvb / (ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(kvb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        rec["splits"] = pkg.paged_prefill_plan(cs.history, 1, cs.n_q_heads, cs.n_kv_heads, cs.head_dim)["n_splits"]
        res[c["name"]] = rec
        del kq, ks, vq, vs, bt
        torch.cuda.empty_cache()
    return res


def copy_calibration(dev):
    """A 1 GiB device copy (known bytes), three times, for counter scaling."""
    import torch
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return 2 * src.numel()


def q8_measurements(chunks, paged, pkg, synth, stream, reps):
    """Each chunk over 8-bit pages of the same shapes (random quants and
    scales), interleaved with the 16-bit paged chunk; a one-row decode step on
    each history, K/V bytes (quants + scales) against HBM peak; and the
    quantizing append of the chunk's rows."""
    import numpy as np
    import torch
    dev = stream.device
    res = {}
    for c in chunks:
        cs = c["case"]
        qc, kq, ks, vq, vs, bt = q8_pages_for(cs, synth, dev)
        o = torch.empty_like(c["q"])
        f8 = lambda: pkg.paged_prefill_attention_q8(c["q"], kq, ks, vq, vs, bt, cs.history, out=o,
                                                    piece_rows=cs.piece_rows, stream=stream)
        f16 = lambda: paged(c)
        for _ in range(3):
            f8()
            f16()
        m8, m16 = timed_pair(f8, f16, reps, stream)
        q1, o1 = c["q"][:1].contiguous(), torch.empty_like(c["q"][:1])
        fd = lambda: pkg.paged_prefill_attention_q8(q1, kq, ks, vq, vs, bt, cs.history, out=o1, stream=stream)
        for _ in range(3):
            fd()
        md = timed(fd, 2 * reps, stream)[0]
        kvb = (cs.history + 1) * cs.n_kv_heads * (cs.head_dim + cs.head_dim // 16) * 2
        # The quantizing append of the chunk's own rows (its K and V are taken
        # from the 16-bit chunk's values at those positions): 16-bit rows read,
        # quants and scales written.
        ctx = cs.history + cs.rows
        kn, vn = c["k"][cs.history:ctx].contiguous(), c["v"][cs.history:ctx].contiguous()
        fa = lambda: pkg.paged_kv_append_q8(kn, vn, kq, ks, vq, vs, bt, cs.history, stream=stream)
        fa()
        ma = timed(fa, 2 * reps, stream)[0]
        ab = 2 * cs.rows * cs.n_kv_heads * (2 * cs.head_dim + cs.head_dim + cs.head_dim // 16)
        res[c["name"]] = {"ms_median": round(m8, 4), "tflops": round(c["flops"] / (m8 * 1e-3) / 1e12, 1),
                          "over_16bit_pages": round(m8 / m16, 3),
                          "decode_1row_ms_median": round(md, 5),
                          "decode_kv_gbs": round(kvb / (md * 1e-3) / 1e9, 1),
                          "decode_hbm_frac": round(kvb / (md * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "append_q8_chunk_ms_median": round(ma, 5),
                          "append_q8_gbs": round(ab / (ma * 1e-3) / 1e9, 1)}
        del kq, vq, ks, vs, bt, o, qc
        torch.cuda.empty_cache()
    return res


def varlen_measurements(pkg, synth, stream, reps):
    """Several sequences in one launch against one call per sequence: a batch
    of 32 decode rows at histories 2K-16K (16/2 heads, d 256, bf16), over
    16-bit and over 8-bit pages, and eight 256-row chunks at 8K-15K (fp16).
    K/V GB/s counts each sequence's keys once."""
    import numpy as np
    import torch
    dev = stream.device
    rng = np.random.default_rng(99)
    batches = {
        "decode_32x1_h2k_16k_bf16": ([(int(h), 1) for h in rng.integers(2048, 16384, size=32)], "bf16"),
        "prefill_8x256_h8k_15k_f16": ([(8192 + 1024 * i, 256) for i in range(8)], "f16"),
    }
    res = {}
    for name, (seqs, dtype) in batches.items():
        case = synth.make_varlen_case(name, seqs, 16, 2, 256, 16, dtype, seed=41)
        dt = torch.float16 if dtype == "f16" else torch.bfloat16

        def dv(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).to(dev)

        q, kp, vp = dv(case.q), dv(case.k_pages), dv(case.v_pages)
        bt = torch.from_numpy(case.block_tables).to(dev)
        cu = torch.from_numpy(case.cu_rows).to(dev)
        hist = torch.from_numpy(case.history_lens).to(dev)
        o, o1 = torch.empty_like(q), torch.empty_like(q)
        rows = [(int(case.cu_rows[i]), int(case.cu_rows[i + 1])) for i in range(len(seqs))]
        qs = [q[a:b] for a, b in rows]
        os_ = [o1[a:b] for a, b in rows]
        bts = [bt[i] for i in range(len(seqs))]
        fv = lambda: pkg.paged_prefill_attention_varlen(q, kp, vp, bt, cu, hist, case.max_rows, case.max_context,
                                                        out=o, stream=stream)

        def fs():
            for i, (h, _) in enumerate(seqs):
                pkg.paged_prefill_attention(qs[i], kp, vp, bts[i], h, out=os_[i], stream=stream)

        for _ in range(3):
            fv()
            fs()
        mv, ms = timed_pair(fv, fs, 2 * reps, stream)
        kvb = sum((h + r) * 2 * 256 * 2 * 2 for h, r in seqs)
        fl = sum(synth.exact_flops(h, r, 16, 256) for h, r in seqs)
        plan = pkg.paged_prefill_plan_varlen(len(seqs), int(case.cu_rows[-1]), case.max_rows, case.max_context,
                                             16, 2, 256)
        res[name] = {"ms_median": round(mv, 5), "one_call_per_sequence_ms_median": round(ms, 5),
                     "speedup_over_separate_calls": round(ms / mv, 3),
                     "kv_gbs": round(kvb / (mv * 1e-3) / 1e9, 1),
                     "hbm_frac": round(kvb / (mv * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "tflops": round(fl / (mv * 1e-3) / 1e12, 1), "splits": plan["n_splits"],
                     # the two plans cut the histories into different splits: rounding differs
                     "max_abs_diff_vs_separate_calls": float((o.float() - o1.float()).abs().max())}
        del q, kp, vp, bt, cu, hist, o, o1, qs, os_, bts
        torch.cuda.empty_cache()
    # The decode batch over 8-bit pages: one launch against one call per
    # sequence; K/V bytes are the quants and scales.
    seqs = batches["decode_32x1_h2k_16k_bf16"][0]
    case = synth.make_varlen_q8_case("decode_q8", seqs, 16, 2, 256, 16, "bf16", seed=43)
    q = torch.from_numpy(np.ascontiguousarray(case.q).view(np.int16)).view(torch.bfloat16).to(dev)
    kq, vq = torch.from_numpy(case.k_quant).to(dev), torch.from_numpy(case.v_quant).to(dev)
    ks = torch.from_numpy(case.k_scale.view(np.int16)).to(dev)
    vs = torch.from_numpy(case.v_scale.view(np.int16)).to(dev)
    bt = torch.from_numpy(case.block_tables).to(dev)
    cu = torch.from_numpy(case.cu_rows).to(dev)
    hist = torch.from_numpy(case.history_lens).to(dev)
    o, o1 = torch.empty_like(q), torch.empty_like(q)
    fv = lambda: pkg.paged_prefill_attention_varlen_q8(q, kq, ks, vq, vs, bt, cu, hist, case.max_rows,
                                                       case.max_context, out=o, stream=stream)

    def fs():
        for i, (h, _) in enumerate(seqs):
            pkg.paged_prefill_attention_q8(q[i:i + 1], kq, ks, vq, vs, bt[i], h, out=o1[i:i + 1], stream=stream)

    for _ in range(3):
        fv()
        fs()
    mv, ms = timed_pair(fv, fs, 2 * reps, stream)
    kvb = sum((h + r) * 2 * (256 + 256 // 16) * 2 for h, r in seqs)
    res["decode_32x1_h2k_16k_bf16_8bit_pages"] = {
        "ms_median": round(mv, 5), "one_call_per_sequence_ms_median": round(ms, 5),
        "speedup_over_separate_calls": round(ms / mv, 3), "kv_gbs": round(kvb / (mv * 1e-3) / 1e9, 1),
        "hbm_frac": round(kvb / (mv * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "max_abs_diff_vs_separate_calls": float((o.float() - o1.float()).abs().max())}
    del q, kq, vq, ks, vs, bt, cu, hist, o, o1
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the work would split by KV head or by history range; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_prefill_amd as pkg
    from paged_kv_prefill_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    names = [c for c in args.chunks.split(",") if c]

    def to_dev(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).to(dev)

    chunks = []
    for name in names:
        case = synth.config_case(name)
        dt = torch.float16 if case.dtype == "f16" else torch.bfloat16
        c = {"name": name, "case": case, "q": to_dev(case.q, dt), "kp": to_dev(case.k_pages, dt),
             "vp": to_dev(case.v_pages, dt), "bt": torch.from_numpy(case.block_table).to(dev),
             "k": to_dev(case.k_contig, dt), "v": to_dev(case.v_contig, dt),
             "flops": synth.exact_flops(case.history, case.rows, case.n_q_heads, case.head_dim)}
        c["out"] = torch.empty_like(c["q"])
        c["out_c"] = torch.empty_like(c["q"])
        chunks.append(c)
        print(f"# {name}: H={case.history} R={case.rows} Hq={case.n_q_heads} Hkv={case.n_kv_heads} "
              f"d={case.head_dim} {case.dtype} pieces={case.piece_rows or case.rows} "
              f"GFLOP={c['flops'] / 1e9:.1f}", file=sys.stderr, flush=True)

    if args.decode_only:
        line = {"mode": "decode_only", "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                "decode_1row": decode_only(chunks, pkg, synth, stream, args.steps, args.warmup)}
        if args.copy_calibration:
            line["copy_calibration_bytes"] = copy_calibration(dev)
        print(json.dumps(line), flush=True)
        return

    def paged(c):
        return pkg.paged_prefill_attention(c["q"], c["kp"], c["vp"], c["bt"], c["case"].history,
                                           out=c["out"], piece_rows=c["case"].piece_rows, stream=stream)

    def contig(c):
        return pkg.contiguous_prefill_attention(c["q"], c["k"], c["v"], c["case"].history, out=c["out_c"],
                                                piece_rows=c["case"].piece_rows, stream=stream)

    for _ in range(args.warmup):
        for c in chunks:
            paged(c)
            if not args.no_ab:
                contig(c)
    torch.cuda.synchronize()

    n = args.steps
    ev = {c["name"]: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
          for c in chunks}
    ev_c = {c["name"]: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for c in chunks}
    paged_ms_total = 0.0
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(n):
        for c in chunks:
            a, b = ev[c["name"]][i]
            a.record(stream)
            paged(c)
            b.record(stream)
            if not args.no_ab:
                a2, b2 = ev_c[c["name"]][i]
                a2.record(stream)
                contig(c)
                b2.record(stream)
        print(f"# step {i + 1}/{n} enqueued", file=sys.stderr, flush=True) if (i + 1) % 10 == 0 else None
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    # The same calls with a cold cache: a 512 MB scratch write (more than the
    # 256 MB Infinity Cache plus the 8 x 4 MB L2) before each call, outside
    # its events, so the call reads its K/V from HBM; in alternating rounds
    # with the same call back to back (warm), so that both meet the same clock.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold, warm_rounds = {}, {}
    for c in chunks:
        cold[c["name"]], warm_rounds[c["name"]] = timed_cold_warm(lambda: paged(c), lambda: scratch.fill_(1), 3,
                                                                   max(2, min(n, 4)), stream)
    del scratch
    torch.cuda.synchronize()

    per_chunk = {}
    for c in chunks:
        ms = np.array([a.elapsed_time(b) for a, b in ev[c["name"]]])
        paged_ms_total += ms.sum()
        cm = cold[c["name"]]
        rec = {"ms_median": float(np.median(ms)), "ms_p10": float(np.percentile(ms, 10)),
               "ms_p90": float(np.percentile(ms, 90)),
               "cold_ms_median": cm[0], "cold_ms_p10": cm[1], "cold_ms_p90": cm[2],
               "warm_alternating_ms_median": warm_rounds[c["name"]][0],
               "tflops": c["flops"] / (np.median(ms) * 1e-3) / 1e12,
               "tflops_cold": c["flops"] / (cm[0] * 1e-3) / 1e12,
               "tflops_4_rows_ctx_convention": stated_flops(c["case"]) / (np.median(ms) * 1e-3) / 1e12,
               "kv_stream_gbs": kv_bytes(c["case"]) / (np.median(ms) * 1e-3) / 1e9,
               "history": c["case"].history, "piece_rows": c["case"].piece_rows or c["case"].rows,
               "heads": f"{c['case'].n_q_heads}/{c['case'].n_kv_heads}", "head_dim": c["case"].head_dim,
               "dtype": c["case"].dtype,
               "plan_splits": pkg.paged_prefill_plan(c["case"].history, c["case"].piece_rows or c["case"].rows,
                                                     c["case"].n_q_heads, c["case"].n_kv_heads,
                                                     c["case"].head_dim)["n_splits"]}
        if not args.no_ab:
            msc = np.array([a.elapsed_time(b) for a, b in ev_c[c["name"]]])
            rec["contiguous_ms_median"] = float(np.median(msc))
            rec["paged_over_contiguous"] = float(np.median(ms) / np.median(msc))
            rec["bitwise_equal_to_contiguous"] = bool(torch.equal(c["out"].view(torch.int16),
                                                                  c["out_c"].view(torch.int16)))
        per_chunk[c["name"]] = rec

    total_flops = sum(c["flops"] for c in chunks)
    step_ms = paged_ms_total / n
    value = total_flops / (step_ms * 1e-3) / 1e12
    value_cold = total_flops / (sum(cold[c["name"]][0] for c in chunks) * 1e-3) / 1e12

    roofline = None
    rc = next((c for c in chunks if c["name"] == ROOFLINE_CHUNK), None)
    if rc is not None:
        plan = pkg.paged_prefill_plan(rc["case"].history, rc["case"].rows, rc["case"].n_q_heads,
                                      rc["case"].n_kv_heads, rc["case"].head_dim)
        assert plan["n_splits"] == 1  # one kernel launch per call: the events bracket exactly it
        ms = np.array([a.elapsed_time(b) for a, b in ev[ROOFLINE_CHUNK]])
        achieved = rc["flops"] / (ms.mean() * 1e-3) / 1e12
        khash = kernel_source_hash()
        traffic = load_traffic(khash)
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["f16"], "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_TFLOPS["f16"], 4), "traffic": traffic,
                    "kernel": "attn_partial_kernel<256, F16, paged> (32K-history 2048-row chunk, one launch)",
                    "launch_ms_mean": round(float(ms.mean()), 4), "kernel_source_hash": khash}
        clock = load_clock(khash)
        if clock:
            # the same peak scaled to the clock the counters saw (at most that clock)
            peak_clk = PEAK_TFLOPS["f16"] * clock / NOMINAL_CLOCK_GHZ
            roofline.update({"clock_ghz_counters": round(clock, 3), "peak_at_that_clock": round(peak_clk, 1),
                             "frac_at_that_clock": round(achieved / peak_clk, 4)})
        pw = load_power(khash)
        if pw and ROOFLINE_CHUNK in pw and "matmul_f16_8192" in pw:
            # under sustained load the board power limit sets the clock: the
            # same chip's fp16 matmul rate is the practical ceiling
            mm, rcp = pw["matmul_f16_8192"], pw[ROOFLINE_CHUNK]
            roofline.update({"sustained_power_w": rcp["power_w_median"],
                             "sustained_clock_mhz": rcp["gfx_clock_mhz_mean"],
                             "matmul_f16_8192_tflops": mm["tflops"], "matmul_power_w": mm["power_w_median"],
                             "matmul_clock_mhz": mm["gfx_clock_mhz_mean"],
                             "frac_of_matmul": round(achieved / mm["tflops"], 4)})

    line = {
        "metric": "paged prefill-attn TFLOP/s + ms per 2048-row chunk at 32K-128K history",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16+bf16 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "one 2048-row chunk each at 32K (16/2 heads, d256, fp16, one call), "
                               "64K (32/4, d128, bf16, 8x256-row pieces) and 128K history (16/2, d256, "
                               "bf16, 16x128-row pieces, pages scattered in a 65536-page pool); paged KV, "
                               "16-token pages in random order",
                   "chunks": per_chunk, "wall_s": round(wall, 3),
                   "value_timing": "the K timed steps back to back (between two calls of a chunk the other "
                                   "chunks and the contiguous A/B calls stream about 550 MB, more than the 256 MB "
                                   "Infinity Cache); value_cold and each chunk's cold_ms_median time the same "
                                   "calls after a 512 MB scratch write, in rounds alternating with the same call "
                                   "back to back (warm_alternating_ms_median)",
                   "value_cold": round(value_cold, 2),
                   "flop_convention": "exact causal: 4 d Hq (R H + R (R + 1) / 2) per call; "
                                      "tflops_4_rows_ctx_convention uses 4 R (H + R) d Hq per call"},
        "roofline": roofline,
    }

    if args.power > 0:
        line["config"]["power"] = power_measurements(chunks, paged, stream, args.power)

    if not args.no_extra:
        print("# extra measurements", file=sys.stderr, flush=True)
        line["config"]["extra"] = extra_measurements(chunks, paged, contig, pkg, synth, to_dev, stream)

    if args.copy_calibration:
        line["copy_calibration_bytes"] = copy_calibration(dev)

    if not args.no_cpu:
        # the roofline chunk first, then the others in step order
        ordered = sorted(chunks, key=lambda c: c["name"] != ROOFLINE_CHUNK)
        line["cpu_baseline"] = cpu_baseline([c["case"] for c in ordered])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
