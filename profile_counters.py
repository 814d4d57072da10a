"""HBM traffic of a kernel from rocprofv3 counters (a measurement aid beside bench.py, not part of
the path).

  copy       run a plain device-to-device copy of a known size (the calibration kernel):
             rocprofv3 --pmc FETCH_SIZE --kernel-include-regex copy -- python3 profile_counters.py copy
  summarize  turn the counter CSVs of the decode kernel and of the copy into
             profiles/<kernel>_<workload>_counters.json: per-launch FETCH_SIZE and WRITE_SIZE, each
             scaled by (true bytes / counted bytes) of the copy, and the hash of the kernel sources
             they were taken on (bench.py reports the traffic only while that hash still matches).
  table      per kernel, the mean per dispatch of every counter in the given CSVs as a markdown
             table: FETCH_SIZE / WRITE_SIZE as calibrated bytes, MfmaUtil in percent,
             SQ_INSTS_VALU_MFMA_MOPS_F16 as fp16 MFMA flops (512 per count), the rest raw.
"""
import argparse
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_MIB = 1024


def run_copy(mib: int, reps: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}", flush=True)


def counter_rows(path_glob: str):
    files = sorted(glob.glob(path_glob, recursive=True))
    if not files:
        raise SystemExit(f"no counter CSV matches {path_glob}")
    rows = []
    for p in files:
        with open(p, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def per_dispatch(rows, kernel_substr: str, counter: str):
    """Mean over dispatches of the summed counter value (KiB for FETCH_SIZE / WRITE_SIZE)."""
    acc = {}
    for r in rows:
        if kernel_substr not in r.get("Kernel_Name", ""):
            continue
        if r.get("Counter_Name") != counter:
            continue
        d = r.get("Dispatch_Id") or r.get("Correlation_Id")
        acc[d] = acc.get(d, 0.0) + float(r["Counter_Value"])
    if not acc:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r}")
    return sum(acc.values()) / len(acc), len(acc)


def summarize(a) -> None:
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash
    kf, nkf = per_dispatch(counter_rows(a.fetch), a.kernel, "FETCH_SIZE")
    kw, nkw = per_dispatch(counter_rows(a.write), a.kernel, "WRITE_SIZE")
    cf, _ = per_dispatch(counter_rows(a.copy_fetch), a.copy_kernel, "FETCH_SIZE")
    cw, _ = per_dispatch(counter_rows(a.copy_write), a.copy_kernel, "WRITE_SIZE")
    true_kib = a.copy_mib * 1024.0
    ff, fw = true_kib / cf, true_kib / cw
    fetch_b, write_b = kf * ff * 1024.0, kw * fw * 1024.0
    out = {
        "kernel": a.kernel, "workload": a.workload,
        "fetch_kib_per_dispatch_raw": round(kf, 1), "write_kib_per_dispatch_raw": round(kw, 1),
        "dispatches": {"fetch": nkf, "write": nkw},
        "copy_calibration": {"copy_mib": a.copy_mib, "fetch_kib_raw": round(cf, 1), "write_kib_raw": round(cw, 1),
                             "fetch_factor": round(ff, 4), "write_factor": round(fw, 4)},
        "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(fetch_b + write_b),
        "source_hash": kernel_source_hash(),
    }
    dst = os.path.join(ROOT, "profiles", f"{a.kernel}_{a.workload}_counters.json")
    with open(dst, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def table(a) -> None:
    rows = []
    for g in a.csv:
        rows.extend(counter_rows(g))
    ff = fw = None
    if a.copy_fetch and a.copy_write:
        cf, _ = per_dispatch(counter_rows(a.copy_fetch), a.copy_kernel, "FETCH_SIZE")
        cw, _ = per_dispatch(counter_rows(a.copy_write), a.copy_kernel, "WRITE_SIZE")
        ff, fw = a.copy_mib * 1024.0 / cf, a.copy_mib * 1024.0 / cw
    # kernel -> counter -> dispatch -> summed value
    acc = {}
    for r in rows:
        k = r.get("Kernel_Name", "")
        if not any(s in k for s in a.kernels):
            continue
        short = next(s for s in a.kernels if s in k)
        d = r.get("Dispatch_Id") or r.get("Correlation_Id")
        c = acc.setdefault(short, {}).setdefault(r["Counter_Name"], {})
        c[d] = c.get(d, 0.0) + float(r["Counter_Value"])
    counters = sorted({c for v in acc.values() for c in v})
    head = ["kernel", "dispatches"]
    for c in counters:
        head.append({"FETCH_SIZE": "fetched MB", "WRITE_SIZE": "written MB", "MfmaUtil": "MFMA busy %",
                     "SQ_INSTS_VALU_MFMA_MOPS_F16": "fp16 MFMA GFLOP"}.get(c, c))
    print("| " + " | ".join(head) + " |")
    print("|" + "---|" * len(head))
    for k in a.kernels:
        if k not in acc:
            continue
        cells = [k, str(max(len(v) for v in acc[k].values()))]
        for c in counters:
            vals = acc[k].get(c)
            if not vals:
                cells.append("")
                continue
            m = sum(vals.values()) / len(vals)
            if c == "FETCH_SIZE" and ff:
                cells.append(f"{m * ff * 1024 / 1e6:.1f}")
            elif c == "WRITE_SIZE" and fw:
                cells.append(f"{m * fw * 1024 / 1e6:.1f}")
            elif c == "MfmaUtil":
                cells.append(f"{m:.1f}")
            elif c == "SQ_INSTS_VALU_MFMA_MOPS_F16":
                cells.append(f"{m * 512 / 1e9:.2f}")
            else:
                cells.append(f"{m:.4g}")
        print("| " + " | ".join(cells) + " |")
    if ff:
        print(f"\nCopy calibration: fetched bytes = {ff:.3f} x FETCH_SIZE KiB x 1024, written = {fw:.3f} x WRITE_SIZE.")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=COPY_MIB)
    c.add_argument("--reps", type=int, default=3)
    s = sub.add_parser("summarize")
    s.add_argument("--kernel", default="decode_kernel")
    s.add_argument("--workload", required=True)
    s.add_argument("--fetch", required=True, help="glob of the kernel's FETCH_SIZE counter CSV(s)")
    s.add_argument("--write", required=True)
    s.add_argument("--copy-kernel", default="copy")
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--copy-mib", type=int, default=COPY_MIB)
    t = sub.add_parser("table")
    t.add_argument("--csv", action="append", required=True, help="glob of counter CSV(s); repeatable")
    t.add_argument("--kernels", nargs="+", required=True, help="kernel name substrings, in table order")
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--copy-fetch")
    t.add_argument("--copy-write")
    t.add_argument("--copy-mib", type=int, default=COPY_MIB)
    a = ap.parse_args()
    if a.cmd == "copy":
        run_copy(a.mib, a.reps)
    elif a.cmd == "table":
        table(a)
    else:
        summarize(a)


if __name__ == "__main__":
    main()
