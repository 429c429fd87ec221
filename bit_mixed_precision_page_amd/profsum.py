"""Turn rocprofv3 CSV output of the decode benchmark into the short text
summaries kept under profiles/.

  python -m bit_mixed_precision_page_amd.profsum trace DIR WORKLOAD "COMMAND"
      DIR holds run_kernel_stats.csv of a --kernel-trace --stats run;
      writes profiles/kernel_trace__WORKLOAD.txt.
  python -m bit_mixed_precision_page_amd.profsum pmc FETCH_DIR WRITE_DIR WORKLOAD "CMD1" "CMD2" COPY_BYTES [KERNEL]
      FETCH_DIR / WRITE_DIR hold run_counter_collection.csv of a --pmc FETCH_SIZE and a
      --pmc WRITE_SIZE run of the benchmark; writes
      profiles/KERNEL__WORKLOAD__pmc.txt (JSON) with the split kernel's HBM
      bytes per launch and the SHA-256 of the sources it was built from
      (KERNEL: decode_split_kernel, the default, or pool_split_kernel).

  python -m bit_mixed_precision_page_amd.profsum sq WORKLOAD KERNEL SIMDS DIR "CMD" [DIR "CMD" ...]
      each DIR holds run_counter_collection.csv of one --pmc pass over SQ
      counters; writes profiles/KERNEL__WORKLOAD__sq.txt (JSON): every
      counter's mean per dispatch of KERNEL, the instruction counts per wave
      and per SIMD (SIMDS = SIMDs of the device), the share of the matrix
      core's busy cycles with a VALU instruction issued beside it, and the
      share of wave time spent waiting to issue.

Counter scaling: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are divided by
what they read for the runtime's device-to-device copy kernel
(__amd_rocclr_copyBuffer) on the benchmark's cache replicas, whose size is
known exactly (one replica per copy, read once and written once; the
benchmark prints it as "replica bytes"); copies of small host transfers,
which the runtime also stages through that kernel, are left out.
"""
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COPY = "__amd_rocclr_copyBuffer"
# sources each profiled kernel is built from: a counter record holds only for that code
KERNEL_SRC = {"decode_split_kernel": ["kvq_internal.h", "kvq_decode_core.h", "kvq_decode.hip"],
              "pool_split_kernel": ["kvq_internal.h", "kvq_decode_core.h", "kvq_pool.hip"],
              "prefill_fwd_kernel": ["kvq_internal.h", "kvq_decode_core.h", "kvq_prefill.hip"]}


def source_sha256(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SRC[kernel]:
        h.update(open(os.path.join(HERE, "csrc", f), "rb").read())
    return h.hexdigest()


def short(name):
    s = name.replace("kvq::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", s)


def trace(d, workload, command):
    path = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(path)))
    lines = ["# rocprofv3 kernel trace summary (durations in microseconds)",
             f"# workload: {workload}",
             f"# command: {command}", "",
             f"{'kernel':<46} {'calls':>6} {'total_us':>11} {'avg_us':>9} {'min_us':>9} "
             f"{'max_us':>9} {'pct':>6}"]
    for r in rows:
        lines.append(f"{short(r['Name']):<46} {int(r['Calls']):>6} "
                     f"{float(r['TotalDurationNs']) / 1e3:>11.1f} "
                     f"{float(r['AverageNs']) / 1e3:>9.2f} {float(r['MinNs']) / 1e3:>9.2f} "
                     f"{float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>6.2f}")
    out = os.path.join(ROOT, "profiles", f"kernel_trace__{workload}.txt")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return out


def counter_means(d, counter, split, copy_kib):
    """Mean counter value per dispatch of the split kernel and of the copy
    kernel's replica copies.  Only copies whose counter reads at least a
    quarter of the replica size count: the runtime also runs its copy kernel
    for small host-to-device transfers through staging memory, which read
    host memory and would dilute the calibration."""
    vals = {split: [], COPY: []}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            for key in vals:
                if key in r["Kernel_Name"]:
                    v = float(r["Counter_Value"])
                    if key == COPY and v < 0.25 * copy_kib:
                        continue
                    vals[key].append(v)
    for key, v in vals.items():
        if not v:
            raise SystemExit(f"no {counter} samples for {key} under {d}")
    return {k: sum(v) / len(v) for k, v in vals.items()}, {k: len(v) for k, v in vals.items()}


def pmc(fetch_dir, write_dir, workload, cmd_fetch, cmd_write, copy_bytes,
        split="decode_split_kernel"):
    copy_kib = copy_bytes / 1024.0
    f, nf = counter_means(fetch_dir, "FETCH_SIZE", split, copy_kib)
    w, nw = counter_means(write_dir, "WRITE_SIZE", split, copy_kib)
    f_scale = copy_kib / f[COPY]
    w_scale = copy_kib / w[COPY]
    fetch_b = f[split] * f_scale * 1024.0
    write_b = w[split] * w_scale * 1024.0
    rec = {
        "kernel": split, "workload": workload,
        "fetch_kib_per_dispatch_raw": round(f[split], 1),
        "write_kib_per_dispatch_raw": round(w[split], 1),
        "copy_kernel": COPY, "copy_bytes": copy_bytes,
        "copy_fetch_kib_raw": round(f[COPY], 1), "copy_write_kib_raw": round(w[COPY], 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "hbm_read_bytes_per_launch": round(fetch_b),
        "hbm_write_bytes_per_launch": round(write_b),
        "hbm_bytes_per_launch": round(fetch_b + write_b),
        "dispatches": {"fetch": nf, "write": nw},
        "commands": [cmd_fetch, cmd_write],
        "source_sha256": source_sha256(split),
    }
    out = os.path.join(ROOT, "profiles", f"{split}__{workload}__pmc.txt")
    open(out, "w").write(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec, indent=1))
    return out


def sq(workload, kernel, simds, passes):
    """passes: [(dir, command)] of --pmc runs over SQ counters."""
    means, counts = {}, {}
    for d, _ in passes:
        per = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                if kernel not in r["Kernel_Name"]:
                    continue
                per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if not per:
            raise SystemExit(f"no {kernel} samples under {d}")
        for c, v in per.items():
            if c in means:
                continue
            means[c] = sum(v) / len(v)
            counts[c] = len(v)
    rec = {"kernel": kernel, "workload": workload, "simds": simds,
           "mean_per_dispatch": {c: round(v, 1) for c, v in sorted(means.items())},
           "dispatches": counts}
    der = {}
    waves = means.get("SQ_WAVES")
    for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS"):
        if c in means:
            der[c + "_per_simd"] = round(means[c] / simds, 1)
            if waves:
                der[c + "_per_wave"] = round(means[c] / waves, 1)
    if "SQ_VALU_MFMA_BUSY_CYCLES" in means:
        der["mfma_busy_cycles_per_simd"] = round(means["SQ_VALU_MFMA_BUSY_CYCLES"] / simds, 1)
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in means:
            der["valu_issued_while_mfma_busy"] = round(
                means["SQ_VALU_MFMA_COEXEC_CYCLES"] / means["SQ_VALU_MFMA_BUSY_CYCLES"], 3)
    if "SQ_WAIT_INST_ANY" in means and "SQ_WAVE_CYCLES" in means:
        der["wave_time_waiting_to_issue"] = round(means["SQ_WAIT_INST_ANY"] / means["SQ_WAVE_CYCLES"], 3)
    rec["derived"] = der
    rec["commands"] = [cmd for _, cmd in passes]
    rec["source_sha256"] = source_sha256(kernel)
    out = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__sq.txt")
    open(out, "w").write(json.dumps(rec, indent=1) + "\n")
    print(json.dumps(rec, indent=1))
    return out


def main(argv):
    if argv[:1] == ["sq"]:
        rest = argv[4:]
        sq(argv[1], argv[2], int(argv[3]), list(zip(rest[0::2], rest[1::2])))
        return
    if argv[:1] == ["trace"]:
        trace(argv[1], argv[2], argv[3])
    elif argv[:1] == ["pmc"]:
        pmc(argv[1], argv[2], argv[3], argv[4], argv[5], int(argv[6]), *argv[7:8])
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
