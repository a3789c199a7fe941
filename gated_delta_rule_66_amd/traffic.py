"""HBM traffic per kernel launch from rocprofv3 counter runs.

Reads the ``counter_collection.csv`` files of rocprofv3 ``--pmc FETCH_SIZE``
and ``--pmc WRITE_SIZE`` runs (``-f csv``): one pair taken over a benchmark
command, one pair over a plain device copy of known size (``bench.py
--copy-probe-mib N``: 5 copies that each read and write N MiB).  The copy
calibrates the counters: factor = known bytes / counted bytes per copy
dispatch, for reads and writes separately.  Writes a JSON record with the
scaled bytes per launch of each library kernel, keyed by the names the library
uses for its launches, together with a hash of the kernel sources (so that a
reader can tell when the record no longer describes the current kernels).

    python -m gated_delta_rule_66_amd.traffic --fetch DIR --write DIR \\
        --copy-fetch DIR --copy-write DIR --copy-mib N --plan NSEG,VB,SPLIT --out FILE
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    """sha256 over the HIP/C++ sources the library is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp", ".inc")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _first_bool(kernel_name: str, after: str):
    """The first bool template argument of a kernel symbol, mangled (Lb0E /
    Lb1E) or demangled (false / true), after the name `after`."""
    n = kernel_name[kernel_name.index(after) + len(after):]
    cands = [(n.find(tok), val) for tok, val in (("Lb0E", False), ("Lb1E", True),
                                                  ("false", False), ("true", True))]
    cands = [c for c in cands if c[0] >= 0]
    return min(cands)[1] if cands else False


def launch_name(kernel_name: str):
    """Library launch name of a kernel symbol (None for other kernels)."""
    n = kernel_name
    if "kda_chunk_kernel" in n:
        # template flag SUMMARY is the first bool template argument
        return "chunk_summary" if _first_bool(n, "kda_chunk_kernel") else "chunk_output"
    if "kda_intra_kernel" in n:
        return "intra_chunk"
    if "kda_state_kernel" in n:
        # <T, K, waves, tiles, SUMMARY, OUT, GATE>
        return "state_summary" if _first_bool(n, "kda_state_kernel") else "state_output"
    if "kda_fused_first_kernel" in n:
        # segment 0 with output beside the summaries: the summary launch
        return "fused_summary"
    if "kda_fused_kernel" in n:
        # <GATE>: the output pass, gated or not
        return "fused_output"
    if "kda_scan_kernel" in n:
        return "segment_scan"
    if "kda_decode_multi_kernel" in n:
        return "decode_steps"
    if "kda_decode_kernel" in n:
        return "decode_step"
    if "kda_copy_state_kernel" in n:
        return "copy_state"
    return None


def read_counter(directory: str, counter: str):
    """[(kernel name, value)] per dispatch of `counter` under `directory`."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under %s" % directory)
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"])))
    return rows


def per_launch(rows):
    acc = {}
    for kname, val in rows:
        ln = launch_name(kname)
        if ln is None:
            continue
        acc.setdefault(ln, []).append(val)
    return {k: sum(v) / len(v) for k, v in acc.items()}


def copy_value(rows):
    """Average counter value per copy dispatch of the calibration run."""
    cp = [v for k, v in rows if "copy" in k.lower()]
    if not cp:
        cp = [v for _, v in rows[-5:]]
    return sum(cp) / len(cp)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--plan", required=True, help="n_seg,v_block,split of the profiled prefill call")
    ap.add_argument("--workload", default="")
    ap.add_argument("--command", default="")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()

    copy_bytes = a.copy_mib * (1 << 20)
    f_copy = copy_value(read_counter(a.copy_fetch, "FETCH_SIZE")) * 1024.0
    w_copy = copy_value(read_counter(a.copy_write, "WRITE_SIZE")) * 1024.0
    f_factor = copy_bytes / f_copy
    w_factor = copy_bytes / w_copy
    fetch = per_launch(read_counter(a.fetch, "FETCH_SIZE"))
    write = per_launch(read_counter(a.write, "WRITE_SIZE"))
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        fb = fetch.get(name, 0.0) * 1024.0 * f_factor
        wb = write.get(name, 0.0) * 1024.0 * w_factor
        kernels[name] = {"fetch_kib_raw": fetch.get(name), "write_kib_raw": write.get(name),
                         "read_bytes": fb, "write_bytes": wb, "hbm_bytes_per_launch": fb + wb}
    rec = {
        "workload": a.workload,
        "plan": [int(x) for x in a.plan.split(",")],
        "source_sha256": kernel_source_hash(),
        "calibration": {"copy_bytes": copy_bytes, "fetch_kib_per_copy": f_copy / 1024.0,
                        "write_kib_per_copy": w_copy / 1024.0, "fetch_factor": f_factor,
                        "write_factor": w_factor},
        "kernels": kernels,
        "command": a.command,
        "note": "FETCH_SIZE / WRITE_SIZE per dispatch scaled by the plain-copy calibration",
    }
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
