"""Summaries of rocprofv3 counter runs: HBM traffic per kernel launch.

Two counter passes over the same command (``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE``, both in KiB per dispatch) are scaled by what the same
counters read, in that run, for kernels of known traffic: ``bench.py
--calibrate`` first runs the library's read-only stream over 256 MiB
(``k_stream_read``: 16-byte loads per lane covering whole 128-byte lines, the
GEMVs' code-load pattern) and a write-only fill of 256 MiB.  The calibration
must share the measured kernel's access pattern: FETCH_SIZE reads the
whole-line stream at half its bytes but a torch reduction over the same
buffer at all of them.  The result is in bytes of HBM traffic.  Usage:

    python3 profiling.py traffic --fetch F.csv --write W.csv --kernel k_stage_b \\
        --name routed_gateup_shared_down --workload resident-stack-30L-e128k8-uniform

prints a Markdown summary and records the figure in profiles/traffic.json,
keyed by name, with the hash of the kernel sources it was taken on (bench.py
reports it only while that hash still matches).
"""
import argparse
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "bit_routed_expert_tf_amd", "csrc")
CAL_BYTES = 256 << 20
# device sources each measured kernel is built from
SOURCES = {
    "k_stage": ["tf_decode.hip", "tf_device.h", "tf_layer.h", "tf_internal.h", "tf_slot_dev.h"],
    "k_gu": ["tf_grouped.hip", "tf_device.h", "tf_layer.h", "tf_internal.h", "tf_slot_dev.h"],
    "k_dn": ["tf_grouped.hip", "tf_device.h", "tf_layer.h", "tf_internal.h", "tf_slot_dev.h"],
}


def source_sha256(kernel):
    """Hash of the device sources the kernel is built from."""
    names = next(v for k, v in SOURCES.items() if kernel.startswith(k))
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _per_dispatch(path, counter, match):
    vals = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            vals.append(float(r["Counter_Value"]))
    return vals


def traffic(args):
    is_read = lambda n: "k_stream_read" in n   # noqa: E731  reads CAL_BYTES
    is_fill = lambda n: "FillFunctor" in n     # noqa: E731  torch fill_: writes CAL_BYTES
    is_kern = lambda n: args.kernel in n       # noqa: E731
    kf = _per_dispatch(args.fetch, "FETCH_SIZE", is_kern)
    kw = _per_dispatch(args.write, "WRITE_SIZE", is_kern)
    cf = _per_dispatch(args.fetch, "FETCH_SIZE", is_read)
    cw = _per_dispatch(args.write, "WRITE_SIZE", is_fill)
    if not (kf and kw and cf and cw):
        sys.exit("missing dispatches: kernel %d/%d, calibration %d/%d" % (len(kf), len(kw), len(cf), len(cw)))
    # the largest calibration dispatches are the 256 MiB ones
    cfk, cwk = max(cf), max(cw)
    sf, sw = CAL_BYTES / (cfk * 1024), CAL_BYTES / (cwk * 1024)
    fetch = sum(kf) / len(kf) * 1024 * sf
    write = sum(kw) / len(kw) * 1024 * sw
    rec = {"workload": args.workload, "kernel": args.kernel, "source_sha256": source_sha256(args.kernel),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "hbm_bytes_per_launch": round(fetch + write), "fetch_scale": round(sf, 4),
           "write_scale": round(sw, 4), "dispatches": [len(kf), len(kw)],
           "calibration": "read-only k_stream_read and write-only torch fill_ of 256 MiB, same run"}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[args.name] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(f"| kernel | dispatches | FETCH_SIZE KiB (avg) | WRITE_SIZE KiB (avg) |\n|---|---|---|---|\n"
          f"| `{args.kernel}` | {len(kf)} / {len(kw)} | {sum(kf) / len(kf):.1f} | {sum(kw) / len(kw):.1f} |\n"
          f"| 256 MiB read (k_stream_read) / write (fill) | {len(cf)} / {len(cw)} | {cfk:.1f} | {cwk:.1f} |\n\n"
          f"Scale factors (known bytes / counter bytes): fetch {sf:.4f}, write {sw:.4f}.\n"
          f"HBM traffic per launch: fetch {fetch / 1e6:.3f} MB + write {write / 1e6:.3f} MB "
          f"= {(fetch + write) / 1e6:.3f} MB.")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--name", required=True)
    t.add_argument("--workload", required=True)
    args = ap.parse_args()
    traffic(args)


if __name__ == "__main__":
    main()
