"""Summarise rocprofv3 CSV output into the short text files kept under
profiles/ (kernel time statistics; HBM traffic from FETCH_SIZE/WRITE_SIZE
counter passes scaled by a copy of known size).

  python -m paged_kv_prefill_amd.profsum stats <kernel_stats.csv> <out.txt> "<command>"
  python -m paged_kv_prefill_amd.profsum traffic <fetch.csv> <write.csv> <out.json> <kernel substring> \
      <copy bytes> "<fetch command>" "<write command>"
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
    h = hashlib.sha256()
    # the attention kernels' sources (the counters in profiles/ are theirs)
    for f in ("attn_kernel.h", "attention.hip", "attention_d64_d128.hip", "attention_d256.hip", "kernels.h"):
        with open(os.path.join(ROOT, "paged_kv_prefill_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
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


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], int(sys.argv[6]), sys.argv[7], sys.argv[8])
    else:
        raise SystemExit(__doc__)
