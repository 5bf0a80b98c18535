"""Summarise rocprofv3 CSV output into the short text files kept under
profiles/ (kernel time statistics; HBM traffic from FETCH_SIZE/WRITE_SIZE
counter passes scaled by a copy of known size).

  python -m paged_kv_prefill_amd.profsum stats <kernel_stats.csv> <out.txt> "<command>"
  python -m paged_kv_prefill_amd.profsum traffic <fetch.csv> <write.csv> <out.json> <kernel substring> \
      <copy bytes> "<fetch command>" "<write command>"
  python -m paged_kv_prefill_amd.profsum counters <counters.csv> <out.txt> <kernel substring> \
      <exact flops per launch> <wave-tiles per launch> <launch us from the kernel trace> "<command>"
  python -m paged_kv_prefill_amd.profsum power <bench output with --power> <out.txt> "<command>"
"""

import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def short(name, width=100):
    name = name.replace("ppa::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    return name if len(name) <= width else name[:width - 3] + "..."


def kernel_source_hash():
    """Hash of everything that decides the device code: every HIP translation
    unit and header under csrc/ and the build's per-file compile options
    (register form, flags).  Counter records in profiles/ carry it and are
    used only while it matches."""
    from paged_kv_prefill_amd import build as _build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_prefill_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    h.update(repr((_build.KERNEL_SOURCES, _build.DEVICE_FLAGS, _build.COMMON[:2], _build.ARCH)).encode())
    return h.hexdigest()[:16]


def stats(csv_path, out_path, command):
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}",
             f"# kernel source hash: {kernel_source_hash()}", "",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10} {'pct':>6}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} {float(r['MinNs']) / 1e3:10.1f} "
                     f"{float(r['MaxNs']) / 1e3:10.1f} {float(r['TotalDurationNs']) / 1e6:10.3f} "
                     f"{float(r['Percentage']):6.2f}  {short(r['Name'])}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_kernel(path):
    out = {}
    for r in csv.DictReader(open(path)):
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic(fetch_csv, write_csv, out_json, kernel_sub, copy_bytes, fetch_cmd, write_cmd):
    fetch = _per_kernel(fetch_csv)
    write = _per_kernel(write_csv)
    copy_kib = copy_bytes / 1024.0
    # the copy of known size: its dispatches are the copyBuffer ones writing about copy_bytes
    cw = [v for v in write.get("__amd_rocclr_copyBuffer", []) if v > 0.5 * copy_kib]
    cf = sorted(fetch.get("__amd_rocclr_copyBuffer", []))[-len(cw):] if cw else []
    if not cw or not cf:
        raise SystemExit("no calibration copy found")
    fetch_scale = copy_kib / (sum(cf) / len(cf))
    write_scale = copy_kib / (sum(cw) / len(cw))
    names = [n for n in fetch if kernel_sub in short(n, 1 << 30)]
    if len(names) != 1:
        raise SystemExit(f"kernel match for {kernel_sub!r}: {names}")
    name = names[0]
    f_kib = sum(fetch[name]) / len(fetch[name])
    w_kib = sum(write[name]) / len(write[name])
    rec = {"kernel": short(name, 200), "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_launch_raw": f_kib, "write_kib_per_launch_raw": w_kib,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "calibration": f"device copy of {copy_bytes} bytes: FETCH_SIZE read {sum(cf) / len(cf):.0f} KiB, "
                          f"WRITE_SIZE {sum(cw) / len(cw):.0f} KiB per dispatch",
           "hbm_bytes_per_launch": (f_kib * fetch_scale + w_kib * write_scale) * 1024.0,
           "fetch_command": fetch_cmd, "write_command": write_cmd,
           "launches": {"fetch": len(fetch[name]), "write": len(write[name])}}
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def _per_kernel_counters(path):
    """{kernel: {counter: [value per dispatch]}}"""
    out = {}
    for r in csv.DictReader(open(path)):
        out.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return out


# MI355X: 256 compute units of 4 SIMDs, 2.4 GHz peak engine clock
SIMDS = 1024
CLOCK_GHZ = 2.4


def counters(csv_path, out_path, kernel_sub, exact_flops, tiles, launch_us, command):
    """MFMA utilisation of one kernel from an SQ/GRBM counter pass: the MFMA
    operations the hardware counted (MOPS counters count 512 flops each)
    against the exact attention flops, the matrix-core busy cycles per SIMD
    against the launch's duration at the peak clock, and instructions per
    (wave, 64-key tile)."""
    per = _per_kernel_counters(csv_path)
    names = [n for n in per if kernel_sub in short(n, 1 << 30)]
    if len(names) != 1:
        raise SystemExit(f"kernel match for {kernel_sub!r}: {names}")
    c = {k: sum(v) / len(v) for k, v in per[names[0]].items()}
    n = len(next(iter(per[names[0]].values())))
    # the counter pass's own dispatch durations (ns), for the clock estimate
    durs = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Kernel_Name"] == names[0]:
            durs[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    pass_ns = sum(durs.values()) / len(durs)
    mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
    counted = mops * 512.0
    busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
    gui = c.get("GRBM_GUI_ACTIVE", 0.0)
    lines = [f"# rocprofv3 counter pass: MFMA utilisation of the attention kernel",
             f"# command: {command}", f"# kernel source hash: {kernel_source_hash()}",
             f"# kernel: {short(names[0], 200)}", f"# dispatches averaged: {n}", ""]
    for k in sorted(c):
        lines.append(f"{k:34s} {c[k]:18.0f}")
    lines.append("")
    lines.append(f"exact attention flops per launch   {exact_flops:18.0f}")
    lines.append(f"MFMA flops counted (MOPS x 512)    {counted:18.0f}  ({counted / exact_flops:.3f} x exact)")
    per_simd = busy / SIMDS
    lines.append(f"MFMA busy cycles per SIMD          {per_simd:18.0f}  ({busy / max(c.get('SQ_INSTS_MFMA', 1), 1):.1f} per MFMA)")
    lines.append(f"launch duration (kernel trace)     {launch_us:18.1f} us = {launch_us * 1e3 * CLOCK_GHZ:.0f} cycles at "
                 f"{CLOCK_GHZ} GHz")
    lines.append(f"MFMA utilisation                   {100.0 * per_simd / (launch_us * 1e3 * CLOCK_GHZ):18.1f} %")
    clock = None
    if gui:
        # GRBM_GUI_ACTIVE counts engine cycles, summed over the 8 XCDs, over a
        # counter window a few microseconds longer than the dispatch: per XCD
        # over the dispatch's duration it bounds the clock the kernel ran at
        # from above (about 1% high for a 1 ms launch).
        clock = gui / 8 / pass_ns
        lines.append(f"GRBM_GUI_ACTIVE / 8 XCDs           {gui / 8:18.0f}  over {pass_ns / 1e3:.1f} us "
                     f"(counter-pass dispatch): clock <= {clock:.2f} GHz")
        lines.append(f"MFMA utilisation at that clock     {100.0 * busy / SIMDS / (pass_ns * clock):18.1f} %")
    if tiles:
        lines.append(f"(wave, 64-key tile) pairs per launch {tiles:16.0f}")
        for k in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
            if k in c:
                lines.append(f"{k + ' per (wave, 64-key tile)':44s} {c[k] / tiles:8.1f}")
        if "SQ_WAVE_CYCLES" in c:
            lines.append(f"{'SQ_WAVE_CYCLES per (wave, 64-key tile)':44s} {c['SQ_WAVE_CYCLES'] / tiles:8.1f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    rec = {"kernel": short(names[0], 200), "kernel_source_hash": kernel_source_hash(), "command": command,
           "mfma_flops_counted": counted, "exact_flops": exact_flops,
           "mfma_busy_cycles_per_simd": per_simd, "counter_pass_dispatch_us": pass_ns / 1e3,
           "clock_ghz_upper_bound": clock}
    with open(os.path.splitext(out_path)[0] + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")


def power(bench_out, out_path, command):
    """Board power and engine clock under sustained load, from the JSON line of
    `bench.py --power SECONDS`: per phase (idle, the fp16 matmul reference, each
    chunk) the median socket power, the mean GFX clock, the rate, and the rate
    as a fraction of the nominal peak and of the matmul's."""
    line = None
    with open(bench_out) as f:
        for l in f:
            if l.startswith("{"):
                line = json.loads(l)
    pw = line["config"]["power"]
    ref = pw.get("matmul_f16_8192", {}).get("tflops")
    lines = ["# board power and engine clock under sustained load (amd-smi metric -p -c, ~0.2 s samples)",
             f"# command: {command}", f"# kernel source hash: {kernel_source_hash()}",
             f"# samples: {pw['samples']}", "",
             f"{'phase':18s} {'power W':>8s} {'GFX MHz':>8s} {'ms/call':>9s} {'TFLOP/s':>8s} "
             f"{'of 2.5 PF':>9s} {'of matmul':>9s}"]
    for name, r in pw.items():
        if not isinstance(r, dict):
            continue
        tf = r.get("tflops")
        lines.append(f"{name:18s} {r['power_w_median'] or 0:8.0f} {r['gfx_clock_mhz_mean'] or 0:8.0f} "
                     f"{r.get('ms_per_call') or 0:9.4f} {tf or 0:8.1f} "
                     f"{(tf or 0) / 2500.0:9.3f} {(tf or 0) / ref if ref else 0:9.3f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    rec = {"kernel_source_hash": kernel_source_hash(), "command": command, "phases": pw}
    with open(os.path.splitext(out_path)[0] + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], int(sys.argv[6]), sys.argv[7], sys.argv[8])
    elif sys.argv[1] == "counters":
        counters(sys.argv[2], sys.argv[3], sys.argv[4], float(sys.argv[5]), float(sys.argv[6]), float(sys.argv[7]),
                 sys.argv[8])
    elif sys.argv[1] == "power":
        power(sys.argv[2], sys.argv[3], sys.argv[4])
    else:
        raise SystemExit(__doc__)
