"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    python -m weight_scans_amd.profiling stats  <kernel_stats.csv>
    python -m weight_scans_amd.profiling traffic <fetch_dir> <write_dir> <config>
    python -m weight_scans_amd.profiling counters <pmc_dir> [<pmc_dir> ...]

`stats` prints a markdown table from a rocprofv3 `--stats` kernel summary CSV
(or a rocpd2summary kernels CSV).  `traffic` reads the counter CSVs of two
`--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of `bench.py`, converts each
counter (KiB per dispatch) into bytes with a scale factor measured on the
plain elementwise kernel (torch.neg over 64 Mi fp32) that bench.py launches
once with a known size (256 MiB read, 256 MiB written), and prints per-pass
HBM traffic.  With --json it also writes
the record bench.py reads back into its roofline `traffic` field, keyed by a
hash of the kernel sources so that a changed kernel invalidates it.
`counters` reads the counter CSVs of `--pmc` runs (SQ_* and GRBM_GUI_ACTIVE,
several runs merged) and prints, per kernel and dispatch, how the matrix
cores, the vector ALU and the LDS were used:
  MFMA busy   SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs):
              the share of all SIMD cycles of the dispatch with an MFMA in
              flight (GRBM_GUI_ACTIVE sums the eight XCDs)
  per wave    SQ_INSTS_MFMA, SQ_INSTS_VALU (MFMA included), SQ_INSTS_LDS
              divided by SQ_WAVES
  LDS conflict  SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS (cycles lost to bank
              conflicts per cycle of LDS issue)
  wait LDS / wait any  SQ_WAIT_INST_LDS and SQ_WAIT_ANY over SQ_WAVE_CYCLES
              (share of the waves' lifetime spent waiting)
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CALIB_BYTES = 256 << 20  # the calibration kernel in bench.py: 256 MiB read + 256 MiB written


def kernel_source_hash() -> str:
    """Hash of every source the library is built from."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        with open(p, "rb") as fh:
            h.update(os.path.basename(p).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    if kernel.startswith(("seg_combine (", "mf_carry (")):  # already a pass-labelled name
        return kernel
    k = kernel
    for pre in ("void ", "gls::(anonymous namespace)::", "at::native::"):
        k = k.replace(pre, "")
    return k.split("(")[0]


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("name")
        calls = int(float(r.get("Calls") or r.get("total_calls")))
        avg = float(r.get("Average (Nsec)") or r.get("AverageNs") or 0) / 1e3
        mn = float(r.get("Min (Nsec)") or r.get("MinNs") or 0) / 1e3
        mx = float(r.get("Max (Nsec)") or r.get("MaxNs") or 0) / 1e3
        pct = float(r.get("Percent (Inc)") or r.get("Percentage") or 0)
        out.append(f"| `{short_name(name)}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f}% |")
    return "\n".join(out)


def _counter(dirpath: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter (summed over dims).
    The segment combine serves both passes: a dispatch of it right after the
    backward's segment pass is named "seg_combine (bwd)", any other one
    "seg_combine (fwd)"."""
    per = defaultdict(float)
    name = {}
    for f in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (f, int(r["Dispatch_Id"]))
            per[key] += float(r["Counter_Value"])
            name[key] = r["Kernel_Name"]
    out = defaultdict(list)
    prev = None
    for key in sorted(per):
        k = name[key]
        if "seg_combine" in k:
            k = "seg_combine (bwd)" if prev is not None and "bwd_lam" in prev else "seg_combine (fwd)"
        if "mf_carry" in k:  # the carry scan of the fp32 / fp64 kernels serves both passes
            k = "mf_carry (bwd)" if prev is not None and "bwd_inc" in prev else "mf_carry (fwd)"
        out[k].append(per[key])
        prev = name[key]
    return dict(out)


def _mean(v):
    return sum(v) / len(v) if v else float("nan")


def counters(dirs):
    """{kernel: {counter: mean per dispatch}} over every counter of the runs."""
    names = set()
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                names.add(r["Counter_Name"])
    res = defaultdict(dict)
    for c in sorted(names):
        for d in dirs:
            for k, v in _counter(d, c).items():
                if v:
                    res[short_name(k)][c] = _mean(v)
    return res


# kernels bench.py itself launches (the read-only cache flush, the fills that
# set up its buffers, the calibration copy): left out of the counter tables
_HARNESS = ("reduce_kernel", "vectorized_elementwise_kernel", "__amd_rocclr")


def counters_table(dirs) -> str:
    res = {k: v for k, v in counters(dirs).items() if not k.startswith(_HARNESS)}
    out = ["| kernel | waves | MFMA busy | MFMA / wave | VALU / wave | LDS / wave | "
           "LDS conflict | wait LDS | wait any |", "|---|---|---|---|---|---|---|---|---|"]

    def ratio(a, b):
        return a / b if b else float("nan")

    for k, c in sorted(res.items()):
        if "GRBM_GUI_ACTIVE" not in c or "SQ_WAVES" not in c:
            continue
        w = c["SQ_WAVES"]
        simd = c["GRBM_GUI_ACTIVE"] / 8.0 * 1024.0
        out.append(
            f"| `{k}` | {w:.0f} | {ratio(c.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0), simd):.3f} | "
            f"{ratio(c.get('SQ_INSTS_MFMA', float('nan')), w):.0f} | "
            f"{ratio(c.get('SQ_INSTS_VALU', float('nan')), w):.0f} | "
            f"{ratio(c.get('SQ_INSTS_LDS', float('nan')), w):.0f} | "
            f"{ratio(c.get('SQ_LDS_BANK_CONFLICT', float('nan')), c.get('SQ_ACTIVE_INST_LDS', 0.0)):.3f} | "
            f"{ratio(c.get('SQ_WAIT_INST_LDS', float('nan')), c.get('SQ_WAVE_CYCLES', 0.0)):.3f} | "
            f"{ratio(c.get('SQ_WAIT_ANY', float('nan')), c.get('SQ_WAVE_CYCLES', 0.0)):.3f} |")
    return "\n".join(out)


def traffic(fetch_dir: str, write_dir: str):
    fetch = _counter(fetch_dir, "FETCH_SIZE")
    write = _counter(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "neg" in k.lower()]
    if not copy:
        raise SystemExit("calibration copy kernel not found in the FETCH_SIZE run")
    # the copy kernel reads and writes CALIB_BYTES; counters are in KiB
    f_scale = CALIB_BYTES / (_mean(fetch[copy[0]]) * 1024.0)
    w_scale = CALIB_BYTES / (_mean(write[copy[0]]) * 1024.0)
    res = {"fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for k in fetch:
        if k not in write:
            continue
        fb = _mean(fetch[k]) * 1024.0 * f_scale
        wb = _mean(write[k]) * 1024.0 * w_scale
        res["kernels"][short_name(k)] = {"fetch_bytes": fb, "write_bytes": wb,
                                         "dispatches": len(fetch[k])}
    return res


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        print(stats_table(argv[1]))
        return 0
    if len(argv) >= 2 and argv[0] == "counters":
        print(counters_table(argv[1:]))
        return 0
    if len(argv) >= 4 and argv[0] == "traffic":
        res = traffic(argv[1], argv[2])
        cfg = argv[3]
        print(f"calibration: FETCH_SIZE x{res['fetch_scale']:.4f}, WRITE_SIZE x{res['write_scale']:.4f}"
              f" (copy kernel, {CALIB_BYTES >> 20} MiB each way)")
        print("| kernel | HBM read (MB) | HBM write (MB) | dispatches |")
        print("|---|---|---|---|")
        for k, v in res["kernels"].items():
            print(f"| `{k}` | {v['fetch_bytes'] / 1e6:.1f} | {v['write_bytes'] / 1e6:.1f} | {v['dispatches']} |")
        if "--json" in argv:
            path = os.path.join(ROOT, "profiles", "traffic.json")
            db = json.load(open(path)) if os.path.exists(path) else {}
            # per-dispatch bytes of every kernel a pass launches once
            def moved(pred):
                return sum(v["fetch_bytes"] + v["write_bytes"] for k, v in res["kernels"].items()
                           if pred(k))
            fwd = moved(lambda k: k.startswith(("fwd_", "qkv_")) or
                        k in ("seg_combine (fwd)", "mf_carry (fwd)"))
            bwd = moved(lambda k: k.startswith("bwd_") or "finalize" in k or
                        k in ("seg_combine (bwd)", "mf_carry (bwd)"))
            db[cfg] = {"kernel_hash": kernel_source_hash(), "fwd_bytes": fwd, "bwd_bytes": bwd,
                       "fetch_scale": res["fetch_scale"], "write_scale": res["write_scale"]}
            with open(path, "w") as fh:
                json.dump(db, fh, indent=1, sort_keys=True)
            print(f"wrote {path}")
        return 0
    print(__doc__)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
